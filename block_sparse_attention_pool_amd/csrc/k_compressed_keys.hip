// Compressed-key (mean-pooled block key) build and incremental update.
//
// K~[b,g,j,:] is the mean of the keys of block j ([SparDA] note,
// prerequisites §3, eq. (4), kernel = stride = 64 tokens).  The cache lives
// on the GPU and is refreshed when tokens are appended (§4.2 step 1, §4.6).
// A touched block is recomputed from all of its keys, so a token-by-token
// update and a bulk build give identical bits.
//
// One workgroup (256 lanes) per (row, touched block): the 64 x d bf16 tile is
// read with 16-byte coalesced loads (a 256-byte key row per 16 lanes at
// d = 128), summed in fp32 per lane, then reduced across the lanes that share
// columns through LDS.  HBM-bound: 64*d*2 bytes read, d*4 bytes written.
#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

template <int D>
__global__ __launch_bounds__(256) void ktilde_kernel(const uint16_t* __restrict__ k,
                                                     float* __restrict__ kt,
                                                     const int32_t* __restrict__ len_old,
                                                     const int32_t* __restrict__ len_new,
                                                     int H_kv, int T_cap, int NB_cap) {
    constexpr int LPR = D / 8;          // lanes per key row (8 bf16 per lane)
    constexpr int RPS = 256 / LPR;      // rows per load step
    constexpr int STEPS = kBlock / RPS;
    __shared__ float red[RPS][D + 4];

    const int row = blockIdx.y;                 // b * H_kv + g
    const int b = row / H_kv;
    int lo = len_old[b];
    int hi = min(len_new[b], T_cap);
    lo = max(lo, 0);
    if (hi <= lo) return;
    const int j = lo / kBlock + (int)blockIdx.x;
    const int j_last = (hi - 1) / kBlock;
    if (j > j_last || j >= NB_cap) return;

    const int t0 = j * kBlock;
    const int n = min(kBlock, hi - t0);         // tokens present in this block
    const int tid = threadIdx.x;
    const int c8 = (tid % LPR) * 8;             // first column of this lane
    const int r0 = tid / LPR;

    const uint16_t* base = k + ((size_t)row * T_cap + t0) * D + c8;
    u32x4 w[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int r = r0 + s * RPS;
        if (r < n) w[s] = ldg16(base + (size_t)r * D);
        else w[s] = u32x4{0, 0, 0, 0};
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += bf16lo(w[s][i]);
            acc[2 * i + 1] += bf16hi(w[s][i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[r0][c8 + i] = acc[i];
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < RPS; ++r) s += red[r][tid];
        kt[((size_t)row * NB_cap + j) * D + tid] = s / (float)n;
    }
}

hipError_t launch_update_compressed_keys(const uint16_t* k, float* kt, const int32_t* len_old,
                                         const int32_t* len_new, int max_blocks_per_row, int B,
                                         int H_kv, int d, int T_cap, int NB_cap, hipStream_t s) {
    dim3 grid(max_blocks_per_row, B * H_kv);
    if (d == 128)
        hipLaunchKernelGGL(ktilde_kernel<128>, grid, dim3(256), 0, s, k, kt, len_old, len_new, H_kv,
                           T_cap, NB_cap);
    else
        hipLaunchKernelGGL(ktilde_kernel<64>, grid, dim3(256), 0, s, k, kt, len_old, len_new, H_kv,
                           T_cap, NB_cap);
    return hipGetLastError();
}

}  // namespace sda
