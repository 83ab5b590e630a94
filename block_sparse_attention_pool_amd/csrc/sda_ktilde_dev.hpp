// Device helpers of the compressed-key (block-mean) update, shared by the
// update launch and the decode step launch: the fp64 -> bf16 rounding and
// the mean of one window of keys by one workgroup.
#pragma once
#include "sda_device.hpp"

namespace sda {

// Nearest bf16 (ties to even) of an fp64 value, rounded once: first to fp32
// by rounding to odd (truncate, then set the last bit if anything was cut),
// which keeps 16 extra bits and a sticky bit, then to nearest even bf16.
// Rounding to odd with two or more extra bits before rounding to nearest
// equals a direct rounding to nearest (Boldo and Melquiond, "Emulation of FMA
// and correctly rounded sums: proved algorithms using rounding to odd").
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    if (x != x) return 0x7FC0;                               // NaN
    const float f = (float)x;                                // nearest; may land past x
    uint32_t u = __float_as_uint(f);
    const double fd = (double)f;
    if (fd != x) {
        if (fabs(fd) > fabs(x)) u -= 1u;                     // one step back toward zero
        u |= 1u;                                             // inexact: odd
    }
    u += 0x7FFFu + ((u >> 16) & 1u);                         // nearest, ties to even
    return (uint16_t)(u >> 16);
}

// Rows of keys one 256-thread load step covers, and the LDS the reduction needs.
template <int D>
struct KtildeShape {
    static constexpr int LPR = D / 8;          // lanes per key row (8 bf16 per lane)
    static constexpr int RPS = 256 / LPR;      // rows per load step
    static constexpr size_t kLdsBytes = (size_t)RPS * (D + 2) * sizeof(double);
};

// Mean of the n (1..64) keys k[row][t0 .. t0+n) stored as entry j of row
// `row` of kt, rounded once to bf16.  Every thread of the workgroup calls it
// (it holds one barrier); threads 0..255 do the work, 16-byte coalesced loads
// summed in fp64 and reduced across the lanes that share columns through
// `red` (KtildeShape<D>::kLdsBytes of LDS).  A sum of bf16 values is exact in
// fp64 while the window's non-zero magnitudes stay within a factor 2^39 of
// each other, so the mean (one correctly rounded fp64 division) and its
// single rounding depend on the keys alone, not on the order of summation.
template <int D>
__device__ __forceinline__ void ktilde_window(const uint16_t* __restrict__ k, uint16_t* __restrict__ kt, int row,
                                              int j, int t0, int n, int T_cap, int NC_cap, int tid,
                                              double (*red)[D + 2]) {
    using S = KtildeShape<D>;
    constexpr int STEPS = kBlock / S::RPS;
    const int c8 = (tid % S::LPR) * 8;          // first column of this lane
    const int r0 = tid / S::LPR;
    if (tid < 256) {
        const uint16_t* base = k + ((size_t)row * T_cap + t0) * D + c8;
        u32x4 w[STEPS];
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int r = r0 + s * S::RPS;
            if (r < n) w[s] = ldg16(base + (size_t)r * D);
            else w[s] = u32x4{0, 0, 0, 0};
        }
        double acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += (double)bf16lo(w[s][i]);
                acc[2 * i + 1] += (double)bf16hi(w[s][i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) red[r0][c8 + i] = acc[i];
    }
    __syncthreads();
    if (tid < D) {
        double s = 0.0;
#pragma unroll
        for (int r = 0; r < S::RPS; ++r) s += red[r][tid];
        kt[((size_t)row * NC_cap + j) * D + tid] = f64_to_bf16(s / (double)n);
    }
}

}  // namespace sda
