// Compressed-key (mean-pooled key) build and incremental update.
//
// K~[b,g,j,:] is the mean of the keys of window j, tokens
// [j*s, min(j*s + l, len)) ([SparDA] note, prerequisites §3, eq. (4) with
// kernel l and stride s: l = s = 64 gives one key per 64-token block; §4.4
// quotes InfLLM-V2's inference setting l = 32, s = 16, overlapping windows).
// The cache lives on the GPU and is refreshed when tokens are appended (§4.2
// step 1, §4.6).  A touched entry is recomputed from all of its keys, so a
// token-by-token update and a bulk build give identical bits.
//
// One workgroup (256 lanes) per (row, touched entry): the <= 64 x d bf16
// tile is read with 16-byte coalesced loads (a 256-byte key row per 16 lanes
// at d = 128), summed in fp64 per lane, then reduced across the lanes that
// share columns through LDS.  A sum of bf16 values is exact in fp64 while the
// window's non-zero magnitudes stay within a factor 2^39 of each other, so
// the mean (one correctly rounded fp64 division) and its single rounding to
// the stored bf16 depend on the keys alone, not on the summation order.
// HBM-bound: l*d*2 bytes read, d*2 bytes written per entry.
#include "sda_device.hpp"
#include "sda_internal.h"
#include "sda_ktilde_dev.hpp"

namespace sda {

template <int D>
__global__ __launch_bounds__(256) void ktilde_kernel(const uint16_t* __restrict__ k,
                                                     uint16_t* __restrict__ kt,
                                                     const int32_t* __restrict__ len_old,
                                                     const int32_t* __restrict__ len_new,
                                                     int H_kv, int T_cap, int NC_cap, int window, int stride) {
    __shared__ double red[KtildeShape<D>::RPS][D + 2];

    const int row = blockIdx.y;                 // b * H_kv + g
    const int b = row / H_kv;
    int lo = len_old[b];
    int hi = min(len_new[b], T_cap);
    lo = max(lo, 0);
    if (hi <= lo) return;
    // entries touched by tokens [lo, hi): windows that end after lo and start before hi
    const int j = (lo >= window ? (lo - window) / stride + 1 : 0) + (int)blockIdx.x;
    const int j_last = (hi - 1) / stride;
    if (j > j_last || j >= NC_cap) return;

    const int t0 = j * stride;
    const int n = min(window, hi - t0);         // tokens present in this window (1..64)
    ktilde_window<D>(k, kt, row, j, t0, n, T_cap, NC_cap, threadIdx.x, red);
}

// Bulk path for overlapping windows (window > stride): a workgroup first sums
// Q consecutive stride-long segments, lane (c, q) adding the s rows of
// segment q in columns 8c .. 8c+7 (16-byte loads; the 16 or 8 lanes of one
// segment read whole key rows), then forms the Q - l/s + 1 windows that lie
// inside those segments, each the sum of l/s consecutive segment sums.
// Every key is read once per workgroup instead of once per window holding it
// (l/s times).  All sums are exact in fp64, so the stored bits equal those
// of ktilde_kernel.
template <int D>
__global__ __launch_bounds__(256) void ktilde_seg_kernel(const uint16_t* __restrict__ k,
                                                         uint16_t* __restrict__ kt,
                                                         const int32_t* __restrict__ len_old,
                                                         const int32_t* __restrict__ len_new,
                                                         int H_kv, int T_cap, int NC_cap, int window, int stride) {
    constexpr int LPR = D / 8;          // lanes per key row (8 bf16 per lane)
    constexpr int Q = 256 / LPR;        // segments per workgroup
    __shared__ double seg[Q][D];

    const int row = blockIdx.y;                 // b * H_kv + g
    const int b = row / H_kv;
    int lo = len_old[b];
    int hi = min(len_new[b], T_cap);
    lo = max(lo, 0);
    if (hi <= lo) return;
    const int per = stride;                     // rows per segment
    const int wins = window / stride;           // segments per window
    const int per_wg = Q - wins + 1;            // windows formed per workgroup
    const int j_lo = lo >= window ? (lo - window) / stride + 1 : 0;
    const int j_last = min((hi - 1) / stride, NC_cap - 1);
    const int e_first = j_lo + (int)blockIdx.x * per_wg;
    if (e_first > j_last) return;

    const int tid = threadIdx.x;
    const int c = tid % LPR;
    const int q = tid / LPR;
    const int t_seg = (e_first + q) * per;      // first token of this lane's segment
    const uint16_t* base = k + ((size_t)row * T_cap) * D + c * 8;
    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    for (int r0 = 0; r0 < per; r0 += 16) {
        u32x4 w[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = t_seg + r0 + r;
            w[r] = (r0 + r < per && t < hi) ? ldg16(base + (size_t)t * D) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += (double)bf16lo(w[r][i]);
                acc[2 * i + 1] += (double)bf16hi(w[r][i]);
            }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) seg[q][c * 8 + i] = acc[i];
    __syncthreads();
    const int j = e_first + q;
    if (q < per_wg && j <= j_last) {
        const int n = min(window, hi - j * stride);      // tokens present in window j
        double sum[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sum[i] = 0.0;
        for (int m = 0; m < wins; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i) sum[i] += seg[q + m][c * 8 + i];
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = (uint32_t)f64_to_bf16(sum[2 * i] / (double)n) |
                   ((uint32_t)f64_to_bf16(sum[2 * i + 1] / (double)n) << 16);
        *reinterpret_cast<u32x4*>(kt + ((size_t)row * NC_cap + j) * D + c * 8) = o;
    }
}

hipError_t launch_update_compressed_keys(const uint16_t* k, uint16_t* kt, const int32_t* len_old,
                                         const int32_t* len_new, int max_entries_per_row, int B,
                                         int H_kv, int d, int T_cap, int NC_cap, int window, int stride,
                                         hipStream_t s) {
    // overlapping windows over a long range: the segment-sum kernel (each key
    // read once); short refreshes: one workgroup per touched window
    if (window > stride && max_entries_per_row > 64) {
        const int q = 256 / (d / 8);
        const int per_wg = q - window / stride + 1;
        dim3 grid((max_entries_per_row + per_wg - 1) / per_wg, B * H_kv);
        if (d == 128)
            hipLaunchKernelGGL(ktilde_seg_kernel<128>, grid, dim3(256), 0, s, k, kt, len_old, len_new, H_kv,
                               T_cap, NC_cap, window, stride);
        else
            hipLaunchKernelGGL(ktilde_seg_kernel<64>, grid, dim3(256), 0, s, k, kt, len_old, len_new, H_kv,
                               T_cap, NC_cap, window, stride);
        return hipGetLastError();
    }
    dim3 grid(max_entries_per_row, B * H_kv);
    if (d == 128)
        hipLaunchKernelGGL(ktilde_kernel<128>, grid, dim3(256), 0, s, k, kt, len_old, len_new, H_kv,
                           T_cap, NC_cap, window, stride);
    else
        hipLaunchKernelGGL(ktilde_kernel<64>, grid, dim3(256), 0, s, k, kt, len_old, len_new, H_kv,
                           T_cap, NC_cap, window, stride);
    return hipGetLastError();
}

}  // namespace sda
