// Device helpers of the top-k selection shared by the scoring launch and the
// decode-step launch: ordered block keys, the key score, bitonic networks
// across lanes, the per-chunk top-k and the final merge of a row's lists.
#pragma once
#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

constexpr int kChunk = 256;          // blocks per scoring workgroup

// ordered 64-bit key: larger score first, then lower block index; 0 = no block
__device__ __forceinline__ uint64_t block_key(float s, int j) {
    return ((uint64_t)float_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

// ---- bitonic networks across the lanes of a wave ------------------------------
// Lane i reads the value of lane i ^ J, all in VALU operations: quad
// permutes (J = 1, 2); row shifts by J up and down, picked by the lane's bit J
// (J = 4, 8); gfx950's swap of adjacent 16-lane rows (J = 16) and of the two
// 32-lane halves (J = 32), whose two results hold the partner's value in the
// lanes of one half each.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
    } else if constexpr (J == 4 || J == 8) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x100 + J, 0xF, 0xF, false);  // lane + J
        const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x110 + J, 0xF, 0xF, false);  // lane - J
        return (__lane_id() & J) ? dn : up;
    } else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (__lane_id() & 16) ? r[0] : r[1];
    } else {
        static_assert(J == 32, "lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (__lane_id() & 32) ? r[0] : r[1];
    }
}
template <int J>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t x) {
    return ((uint64_t)lane_xor<J>((uint32_t)(x >> 32)) << 32) | lane_xor<J>((uint32_t)x);
}

// compare-exchange with lane ^ J: the lane keeps the larger value if
// keep_max, else the smaller
template <int J, typename T>
__device__ __forceinline__ T cmp_xchg(T v, bool keep_max) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit keys");
    T p;
    if constexpr (sizeof(T) == 8) p = (T)lane_xor64<J>((uint64_t)v);
    else p = (T)lane_xor<J>((uint32_t)v);
    return ((p > v) == keep_max) ? p : v;
}

// Sort each aligned segment of P lanes (P a power of two <= 64), largest
// first if DESC, else smallest first.  Stage (k, j): blocks of k lanes
// alternate direction until the last, which takes the segment's direction.
template <int P, bool DESC, int k = 2, typename T>
__device__ __forceinline__ T bitonic_sort(T v, int lane) {
    // the lane masks of the stages are cheap to recompute: keep the compiler
    // from hoisting them into long-lived scalar registers
    if constexpr (k == 2) asm volatile("" : "+v"(lane));
    if constexpr (k <= P) {
        const bool blk = (k == P) ? DESC : (((lane & k) == 0) == DESC);
        if constexpr (k / 2 >= 32) v = cmp_xchg<32>(v, ((lane & 32) == 0) == blk);
        if constexpr (k / 2 >= 16) v = cmp_xchg<((k / 2) >= 32 ? 16 : k / 2 >= 16 ? 16 : 1)>(v, ((lane & 16) == 0) == blk);
        if constexpr (k / 2 >= 8) v = cmp_xchg<8>(v, ((lane & 8) == 0) == blk);
        if constexpr (k / 2 >= 4) v = cmp_xchg<4>(v, ((lane & 4) == 0) == blk);
        if constexpr (k / 2 >= 2) v = cmp_xchg<2>(v, ((lane & 2) == 0) == blk);
        v = cmp_xchg<1>(v, ((lane & 1) == 0) == blk);
        return bitonic_sort<P, DESC, 2 * k>(v, lane);
    } else {
        return v;
    }
}

// Sort a bitonic sequence held by each aligned segment of P lanes, largest first.
template <int P, typename T>
__device__ __forceinline__ T bitonic_merge_desc(T v, int lane) {
    asm volatile("" : "+v"(lane));
    if constexpr (P >= 64) v = cmp_xchg<32>(v, (lane & 32) == 0);
    if constexpr (P >= 32) v = cmp_xchg<16>(v, (lane & 16) == 0);
    if constexpr (P >= 16) v = cmp_xchg<8>(v, (lane & 8) == 0);
    if constexpr (P >= 8) v = cmp_xchg<4>(v, (lane & 4) == 0);
    if constexpr (P >= 4) v = cmp_xchg<2>(v, (lane & 2) == 0);
    if constexpr (P >= 2) v = cmp_xchg<1>(v, (lane & 1) == 0);
    return v;
}

// Score of one pooled key against a vector slice: lane li of each 16-lane row
// holds EPL consecutive dims of both; fused multiply-adds in dim order, then
// the sum over the 16 lanes.  Every scoring path uses it, so their scores
// agree bit for bit.
template <int EPL>
__device__ __forceinline__ float key_dot(const float (&fv)[EPL], const uint32_t* kp) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) {
        acc = fmaf(fv[2 * i], bf16lo(kp[i]), acc);
        acc = fmaf(fv[2 * i + 1], bf16hi(kp[i]), acc);
    }
    return row16_sum(acc);
}

// Level 1 of the selection for one 256-block chunk, by a group of four waves
// (thread t = 0..255 of the group; the group may be part of a larger
// workgroup): sc[t] is the score of block j0 + t; the chunk's K <= 64 best
// keys among blocks in [lo, hi), largest first and zero-padded, go to
// dst[0..K) with agent-scope stores.  Each wave sorts its 64 keys with a
// bitonic network; the four sorted lists merge pairwise (the top 64 of two
// descending lists is the lane-wise max of one and the other reversed, a
// bitonic sequence).  Every thread of the workgroup calls it (three
// workgroup barriers); groups without a chunk pass active = false.
// LDS per group: wl, 4 * 64 keys.
__device__ __forceinline__ void chunk_top_k(const float* sc, int j0, int lo, int hi, int K, bool active,
                                            uint64_t* wl, uint64_t* dst, int t) {
    const int lane = t % kWave, wave = t / kWave;
    const int j = j0 + t;
    uint64_t v = 0;
    if (active) {                                      // uniform over the wave
        const bool valid = j >= lo && j < hi;
        v = bitonic_sort<kWave, true>(valid ? block_key(sc[t], j) : 0ull, lane);
        if (wave & 1) wl[wave * kWave + lane] = v;
    }
    __syncthreads();
    if (active && !(wave & 1)) {
        const uint64_t p = wl[(wave + 1) * kWave + (kWave - 1 - lane)];
        v = bitonic_merge_desc<kWave>(v > p ? v : p, lane);
        if (wave == 2) wl[2 * kWave + lane] = v;
    }
    __syncthreads();
    if (active && wave == 0) {
        const uint64_t p = wl[2 * kWave + (kWave - 1 - lane)];
        v = bitonic_merge_desc<kWave>(v > p ? v : p, lane);
        if (lane < K) __hip_atomic_store(dst + lane, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();                            // wl free for the next chunk
}

// Level 2 of the selection for one row: the nch chunk lists of the row (K
// keys each, descending, at `src`) are padded to P = 2^ceil(log2 K) keys and
// merged pairwise, round by round (one P-lane segment of a wave per pair, a
// bitonic merge of the lane-wise max of one list and the other reversed);
// then one wave sorts the kk selected block ids ascending and the row's block
// set init U top-k U local is written, padded with -1.  Every thread of the
// workgroup calls it (workgroup barriers).  `coherent`: the lists were
// written in this launch by other workgroups (agent-scope loads).
// LDS: bufA nch * P keys, bufB ceil(nch / 2) * P keys (P <= 64).
template <int P, bool coherent>
__device__ __forceinline__ void finish_row_p(const SelectArgs& s, const uint64_t* src, int nch, int vrow, int nb,
                                             uint64_t* bufA, uint64_t* bufB) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, W = blockDim.x / kWave;
    const int K = s.top_k;
    const int lo = min(s.n_init, nb);                      // candidates are [lo, hi)
    const int hi = max(lo, nb - s.n_local);
    const int kk = min(K, hi - lo);
    for (int i = tid; i < nch * P; i += blockDim.x) {
        const int c = i / P, p = i - c * P;
        uint64_t x = 0;
        if (p < K) x = coherent ? __hip_atomic_load(src + c * K + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : src[c * K + p];
        bufA[i] = x;
    }
    __syncthreads();
    uint64_t* cur = bufA;
    uint64_t* nxt = bufB;
    constexpr int SPW = kWave / P;                         // pairs per wave and pass
    const int seg = lane / P, i = lane % P;
    for (int nl = nch; nl > 1; nl = (nl + 1) >> 1) {
        const int np = (nl + 1) >> 1;                      // an odd last list passes through unchanged
        for (int base = wave * SPW; base < np; base += W * SPW) {
            const int m = base + seg;
            const bool ok = m < np;
            const uint64_t x = ok ? cur[2 * m * P + i] : 0ull;
            const uint64_t y = (ok && 2 * m + 1 < nl) ? cur[(2 * m + 1) * P + (P - 1 - i)] : 0ull;
            const uint64_t v = bitonic_merge_desc<P>(x > y ? x : y, lane);
            if (ok) nxt[m * P + i] = v;
        }
        __syncthreads();
        uint64_t* t = cur; cur = nxt; nxt = t;
    }
    int32_t* out = s.block_idx + (size_t)vrow * s.n_sel_max;
    if (wave == 0 && kk > 0) {                             // top-k ids, ascending
        uint32_t id = lane < kk ? 0xFFFFFFFFu - (uint32_t)cur[lane] : 0xFFFFFFFFu;
        id = bitonic_sort<kWave, false>(id, lane);
        if (lane < kk) out[lo + lane] = (int)id;
    }
    for (int i2 = tid; i2 < lo; i2 += blockDim.x) out[i2] = i2;                    // initial blocks
    for (int i2 = tid; i2 < nb - hi; i2 += blockDim.x) out[lo + kk + i2] = hi + i2;  // local blocks
    const int total = lo + kk + (nb - hi);
    for (int p = total + tid; p < s.n_sel_max; p += blockDim.x) out[p] = -1;
    if (tid == 0) s.n_sel[vrow] = total;
    __syncthreads();                                       // bufA / bufB may be reused
}

template <bool coherent>
__device__ __forceinline__ void finish_row(const SelectArgs& s, const uint64_t* src, int nch, int vrow, int nb,
                                           uint64_t* bufA, uint64_t* bufB) {
    switch (pow2_at_least(s.top_k)) {
        case 1: finish_row_p<1, coherent>(s, src, nch, vrow, nb, bufA, bufB); break;
        case 2: finish_row_p<2, coherent>(s, src, nch, vrow, nb, bufA, bufB); break;
        case 4: finish_row_p<4, coherent>(s, src, nch, vrow, nb, bufA, bufB); break;
        case 8: finish_row_p<8, coherent>(s, src, nch, vrow, nb, bufA, bufB); break;
        case 16: finish_row_p<16, coherent>(s, src, nch, vrow, nb, bufA, bufB); break;
        case 32: finish_row_p<32, coherent>(s, src, nch, vrow, nb, bufA, bufB); break;
        default: finish_row_p<64, coherent>(s, src, nch, vrow, nb, bufA, bufB); break;
    }
}

}  // namespace sda
