// Offloaded-KV gather: copy the K/V rows of selected blocks from pinned
// host memory to a compact device staging buffer with GPU loads over the host
// link ([SparDA] note §4.2 steps 3 and 6, §4.5: the selected blocks of the
// next layer are fetched while the current layer computes, and the fetch is
// driven by the GPU rather than by the CPU).
//
// One workgroup per selected entry (grid-strided under a workgroup budget,
// so the copy occupies a bounded share of the CUs while attention runs on
// the others).  Each entry is two 16 KB contiguous row ranges at d = 128;
// 256 lanes move them with 16-byte loads and stores.
#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

template <int D>
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ ksrc,
                                                     const uint16_t* __restrict__ vsrc,
                                                     const int32_t* __restrict__ block_idx,
                                                     const int32_t* __restrict__ n_sel,
                                                     int n_sel_max, int T_cap, int total,
                                                     uint16_t* __restrict__ kst,
                                                     uint16_t* __restrict__ vst,
                                                     int32_t* __restrict__ slot_out) {
    constexpr int CHUNKS = kBlock * D / 8;     // 16-byte chunks per block
    constexpr int CPR = D / 8;                 // chunks per token row
    for (int task = blockIdx.x; task < total; task += gridDim.x) {
        const int row = task / n_sel_max;
        const int e = task - row * n_sel_max;
        const int n = n_sel[row];
        const int j = (e < n) ? block_idx[(size_t)row * n_sel_max + e] : -1;
        const bool ok = (e < n) && j >= 0 && (size_t)j * kBlock < (size_t)T_cap;
        if (threadIdx.x == 0) slot_out[(size_t)row * n_sel_max + e] = ok ? e : -1;
        if (!ok) continue;
        const int rows_avail = min(kBlock, T_cap - j * kBlock);
        const size_t src = ((size_t)row * T_cap + (size_t)j * kBlock) * D;
        const size_t dst = ((size_t)row * n_sel_max * kBlock + (size_t)e * kBlock) * D;
        u32x4 kr[CHUNKS / 256], vr[CHUNKS / 256];
#pragma unroll
        for (int i = 0; i < CHUNKS / 256; ++i) {
            const int c = threadIdx.x + i * 256;
            if (c / CPR < rows_avail) {
                kr[i] = ldg16(ksrc + src + (size_t)c * 8);
                vr[i] = ldg16(vsrc + src + (size_t)c * 8);
            } else {
                kr[i] = u32x4{0, 0, 0, 0};
                vr[i] = u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int i = 0; i < CHUNKS / 256; ++i) {
            const int c = threadIdx.x + i * 256;
            *reinterpret_cast<u32x4*>(kst + dst + (size_t)c * 8) = kr[i];
            *reinterpret_cast<u32x4*>(vst + dst + (size_t)c * 8) = vr[i];
        }
    }
}

hipError_t launch_gather(const uint16_t* k_src, const uint16_t* v_src, const int32_t* block_idx,
                         const int32_t* n_sel, int n_sel_max, int B, int H_kv, int d, int T_cap,
                         uint16_t* k_stage, uint16_t* v_stage, int32_t* slot_out,
                         int max_workgroups, hipStream_t s) {
    const int total = B * H_kv * n_sel_max;
    int grid = total;
    if (max_workgroups > 0 && grid > max_workgroups) grid = max_workgroups;
    if (d == 128)
        hipLaunchKernelGGL(gather_kernel<128>, dim3(grid), dim3(256), 0, s, k_src, v_src, block_idx,
                           n_sel, n_sel_max, T_cap, total, k_stage, v_stage, slot_out);
    else
        hipLaunchKernelGGL(gather_kernel<64>, dim3(grid), dim3(256), 0, s, k_src, v_src, block_idx,
                           n_sel, n_sel_max, T_cap, total, k_stage, v_stage, slot_out);
    return hipGetLastError();
}

}  // namespace sda
