// Device helpers shared by the gfx950 kernels: bf16 storage, vector types,
// wave64 cross-lane reductions (DPP inside a 16-lane row, row swaps across
// rows) and the 16x16x32 bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sda {

constexpr int kBlock = 64;       // tokens per block
constexpr int kWave = 64;        // wavefront width on CDNA

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f2bf(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return f2bf(lo) | (f2bf(hi) << 16);
}

// ---- DPP reductions inside a 16-lane row -----------------------------------
// quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_ror:4 = 0x124,
// row_ror:8 = 0x128.  After the four steps every lane of the row holds the
// row's total.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x124>(x);
    x += dpp_f<0x128>(x);
    return x;
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x124>(x));
    x = fmaxf(x, dpp_f<0x128>(x));
    return x;
}

// max / sum over the four lanes {l, l^16, l^32, l^48}, with the gfx950 row
// swaps (VALU, no LDS round trip): permlane16_swap(x, x) hands lane l the
// pair (value of the even row, value of the odd row) of its two 16-lane rows,
// permlane32_swap the pair of its two 32-lane halves, so each step combines
// the two entries of the pair.  The pair is the same two values on both
// lanes, so every lane of the four ends with the same bits.
__device__ __forceinline__ float cross4_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float cross4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- MFMA -------------------------------------------------------------------
// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies
// A[l % 16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l % 16]; it receives
// D[4*(l/16) + i][l % 16], i = 0..3.
__device__ __forceinline__ floatx4 mfma16x16x32(const u32x4& a, const u32x4& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Registers of a 16-row MFMA A tile (m-tile mt) loaded in whole 128-byte
// lines.  Load kf[mt][2h + x] holds, in lane l, tile row 8x + l%8 (the
// tile's row order: tok_of in the decode, consecutive keys elsewhere) and
// the 16-byte piece (l/16) + 4 ((l/8) % 2) of that row's line h, so every
// load reads 8 whole lines.  (The direct A-layout load reads 64 bytes from
// each of 16 rows, so two loads fetch halves of each line; it streamed up to
// 1.3x slower once a wave walks more than one tile.)  The A layout wants
// lane l to hold tile row l%16 and piece 4k + l/16 of line h in
// kf[mt][2h + k].  Lanes with l%16 < 8 of load x = 0 and lanes with
// l%16 >= 8 of load x = 1 already do; the other halves trade places with the
// lane 8 apart in the same 16-lane row (DPP row rotation by 8, write-masked
// to lane groups 2-3 or 0-1 of each row).
// kswap1 exchanges one m-tile's registers, kswap the four of a 64-row tile.
template <int KS>
__device__ __forceinline__ void kswap1(u32x4 (&kf)[KS]) {
#pragma unroll
    for (int h = 0; h < KS / 2; ++h) {
        const u32x4 a = kf[2 * h], b = kf[2 * h + 1];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            kf[2 * h][c] = (uint32_t)__builtin_amdgcn_update_dpp((int)a[c], (int)b[c], 0x128, 0xF, 0xC, false);
            kf[2 * h + 1][c] = (uint32_t)__builtin_amdgcn_update_dpp((int)b[c], (int)a[c], 0x128, 0xF, 0x3, false);
        }
    }
}
template <int KS>
__device__ __forceinline__ void kswap(u32x4 (&kf)[4][KS]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) kswap1<KS>(kf[mt]);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ldg16_cached(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// A workgroup's arrival at a counter shared by the workgroups of one row,
// made by one thread (thread 0): a relaxed agent-scope increment, returning
// the count before it.  Publication: everything a workgroup hands over (split
// partials, per-chunk candidate lists) is written with agent-scope atomic
// stores, which gfx950 writes through the XCD's non-coherent L2 to the
// agent's coherence point and reports complete (vmcnt) only once they are
// visible there; every wave waits for its own stores to complete
// (s_waitcnt vmcnt(0)) before the workgroup barrier that precedes the
// increment, so all of them are visible to the whole agent before it is
// issued.  A release fence at agent scope would add an L2 write-back
// (buffer_wbl2) that these stores do not need; it doubled the decode step's
// time (46 against 24.7 us at the 128K workload).  Consumption: the arrival
// that sees the final count calls acquire_agent() (L2 invalidate,
// buffer_inv; +0.25 us per step) before the barrier that lets its waves read
// the other workgroups' stores, which they read with agent-scope atomic loads.
__device__ __forceinline__ int arrive(int* counter) {
    return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// 16 bytes stored at byte offset `off` of a region that starts at the
// wave-uniform `base`, with the same device-scope cache bit (sc1, written
// through to the coherence point) as the agent-scope atomic stores above,
// through a buffer store so that the compiler sees the store (and keeps its
// data registers intact until the store has read them).
__device__ __forceinline__ void st_agent16(void* base, uint32_t off, floatx4 v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 16);
}

// order-preserving map float -> uint32 (larger float -> larger key); -0 == +0
__device__ __forceinline__ uint32_t float_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace sda
