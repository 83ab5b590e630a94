// Device helpers of the top-k selection shared by the scoring launch and the
// decode launch that finishes the next layer's selection: ordered block keys,
// wave ranks, sorted-list merges and the final merge of a row's chunk lists.
#pragma once
#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

constexpr int kChunk = 256;          // blocks per scoring workgroup

// ordered 64-bit key: larger score first, then lower block index; 0 = no block
__device__ __forceinline__ uint64_t block_key(float s, int j) {
    return ((uint64_t)float_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

// number of keys larger than `key` among the 64 lanes of the wave: the keys
// travel once round the wave through register rotations
__device__ __forceinline__ int wave_rank(uint64_t key) {
    uint32_t hi = (uint32_t)(key >> 32), lo = (uint32_t)key;
    int r = 0;
#pragma unroll
    for (int i = 1; i < kWave; ++i) {
        hi = wave_ror1(hi);
        lo = wave_ror1(lo);
        r += ((((uint64_t)hi) << 32) | lo) > key;
    }
    return r;
}

// number of keys larger than x in the descending list L[0..len), 1 <= len <= 64:
// the last key of each full 8-key segment tells how many whole segments are
// larger, then the next segment is counted; two rounds of independent reads
__device__ __forceinline__ int count_larger(const uint64_t* L, int len, uint64_t x) {
    uint64_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = L[min(8 * i + 7, len - 1)];      // all reads in bounds, issued together
    int seg = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) seg += (int)((8 * i + 7 < len) & (v[i] > x));
    const int base = 8 * seg;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = L[min(base + i, len - 1)];
    int n = base;
#pragma unroll
    for (int i = 0; i < 8; ++i) n += (int)((base + i < len) & (v[i] > x));
    return n;
}

// One round of pairwise merges over the workgroup: lists c < nl of `len`
// descending keys (zero-padded, len >= K) at src + c * ss; the pair
// (2m, 2m+1) becomes list m of its K largest keys at dst + m * ds.  The list
// strides are odd numbers of keys so that lists start in different LDS banks.  A key's
// place in the merged list is its place in its own list plus the number of
// larger keys in the partner list; keys are distinct apart from the zero
// padding, whose writes may coincide but carry the same value.
// `t` and `nt`: this thread's index among the nt threads that share the round.
__device__ __forceinline__ void merge_round(const uint64_t* src, int nl, int len, int ss, uint64_t* dst, int ds,
                                            int K, int t, int nt) {
    const int items = nl * K;                              // only the first K of a list can stay
    for (int i = t; i < items; i += nt) {
        const int c = i / K, p = i - c * K;
        const uint64_t x = src[c * ss + p];
        int pos = p;
        if ((c ^ 1) < nl) pos += count_larger(src + (c ^ 1) * ss, len, x);
        if (pos < K) dst[(c >> 1) * ds + pos] = x;
    }
}

// Level 2 of the selection for one row: merge the nch sorted chunk lists of
// the row (K = top_k keys each, at `src`) pairwise, round by round, and write
// the row's block set init U top-k U local, ascending, padded with -1.  Every
// thread of the workgroup calls it (it holds barriers).  `coherent`: the lists
// were written in this launch by other workgroups (agent-scope loads).
// LDS: bufA (K|1)*nch keys, bufB (K|1)*ceil(nch/2) keys, sel_j kFusedTopK ints.
template <bool coherent>
__device__ __forceinline__ void finish_row(const SelectArgs& s, const uint64_t* src, int nch, int vrow, int nb,
                                           uint64_t* bufA, uint64_t* bufB, int* sel_j) {
    const int tid = threadIdx.x;
    const int K = s.top_k;
    const int KS = K | 1;
    const int lo = min(s.n_init, nb);                      // candidates are [lo, hi)
    const int hi = max(lo, nb - s.n_local);
    const int kk = min(K, hi - lo);
    for (int i = tid; i < nch * K; i += blockDim.x) {
        const int c = i / K;
        bufA[c * KS + (i - c * K)] =
            coherent ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : src[i];
    }
    __syncthreads();
    uint64_t* cur = bufA;
    uint64_t* nxt = bufB;
    for (int nl = nch; nl > 1; nl = (nl + 1) >> 1) {
        merge_round(cur, nl, K, KS, nxt, KS, K, tid, blockDim.x);
        __syncthreads();
        uint64_t* t = cur; cur = nxt; nxt = t;
    }
    if (tid < kk) sel_j[tid] = (int)(0xFFFFFFFFu - (uint32_t)cur[tid]);
    __syncthreads();
    int32_t* out = s.block_idx + (size_t)vrow * s.n_sel_max;
    for (int i = tid; i < lo; i += blockDim.x) out[i] = i;                   // initial blocks
    if (tid < kk) {                                                          // top-k, ascending
        const int jt = sel_j[tid];
        int pos = 0;
#pragma unroll
        for (int u = 0; u < kFusedTopK; u += 4) {
            const int4 q = *reinterpret_cast<const int4*>(sel_j + u);
            pos += (u + 0 < kk && q.x < jt) + (u + 1 < kk && q.y < jt) +
                   (u + 2 < kk && q.z < jt) + (u + 3 < kk && q.w < jt);
        }
        out[lo + pos] = jt;
    }
    for (int i = tid; i < nb - hi; i += blockDim.x) out[lo + kk + i] = hi + i;  // local blocks
    const int total = lo + kk + (nb - hi);
    for (int p = total + tid; p < s.n_sel_max; p += blockDim.x) out[p] = -1;
    if (tid == 0) s.n_sel[vrow] = total;
    __syncthreads();                                       // bufA / sel_j may be reused
}

// Level 2 for one row by a single wave, with no workgroup barrier (the other
// waves of the workgroup go on with their own work): the row's nch chunk
// lists (K keys each, stride K) are already in LDS at `lists`; `tmp` holds
// ceil(nch/2) * K keys, `sel_j` kFusedTopK ints.  Same block set as finish_row.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's LDS writes are visible to its lanes
}

__device__ __forceinline__ void finish_row_wave(const SelectArgs& s, uint64_t* lists, uint64_t* tmp, int* sel_j,
                                                int nch, int vrow, int nb, int lane) {
    const int K = s.top_k;
    const int lo = min(s.n_init, nb);
    const int hi = max(lo, nb - s.n_local);
    const int kk = min(K, hi - lo);
    uint64_t* cur = lists;
    uint64_t* nxt = tmp;
    for (int nl = nch; nl > 1; nl = (nl + 1) >> 1) {
        merge_round(cur, nl, K, K, nxt, K, K, lane, kWave);
        wave_lds_sync();
        uint64_t* t = cur; cur = nxt; nxt = t;
    }
    if (lane < kk) sel_j[lane] = (int)(0xFFFFFFFFu - (uint32_t)cur[lane]);
    wave_lds_sync();
    int32_t* out = s.block_idx + (size_t)vrow * s.n_sel_max;
    for (int i = lane; i < lo; i += kWave) out[i] = i;
    if (lane < kk) {
        const int jt = sel_j[lane];
        int pos = 0;
#pragma unroll
        for (int u = 0; u < kFusedTopK; u += 4) {
            const int4 q = *reinterpret_cast<const int4*>(sel_j + u);
            pos += (u + 0 < kk && q.x < jt) + (u + 1 < kk && q.y < jt) +
                   (u + 2 < kk && q.z < jt) + (u + 3 < kk && q.w < jt);
        }
        out[lo + pos] = jt;
    }
    for (int i = lane; i < nb - hi; i += kWave) out[lo + kk + i] = hi + i;
    const int total = lo + kk + (nb - hi);
    for (int p = total + lane; p < s.n_sel_max; p += kWave) out[p] = -1;
    if (lane == 0) s.n_sel[vrow] = total;
}

}  // namespace sda
