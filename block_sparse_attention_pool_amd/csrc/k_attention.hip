// Block-sparse decode attention and SSV-style grouped verification.
//
// Computes, for every query head, softmax(q K_B^T * scale) V_B over the
// 64-token blocks of its block list ([SparDA] note eq. (7), §4.2 step 4;
// [SSV] note, NSA selection-branch step 3).  The list is split across
// workgroups (split-K); each wave keeps the online-softmax state (m, l, o)
// of the [SSV] note's online-softmax section, the waves of a workgroup merge
// through LDS, and the last workgroup of a row to finish merges the splits
// by log-sum-exp (no second launch).
//
// Grouped mode ([SSV] core mechanism 1, verification-kernel algorithm): a
// workgroup serves the C*G query heads of a group of C consecutive queries
// that share one KV head.  Exact mode walks the union of the C block lists
// (each block read once) and masks every query to its own list; shared mode
// walks the first query's list for all C queries.  Plain decode is the same
// engine with C = 1.
//
// Tile engine (one wave, one 64-token block; rows = the C*G query heads,
// padded to 16 or 32):
//   S^T[tok][row] = K[tok][:] . Q[row][:]    16x16x32 bf16 MFMA.  K is the A
//       operand, loaded from HBM in whole 128-byte lines (16-byte loads,
//       rows past the sequence end clamped, no branches) and brought into
//       MFMA layout by one DPP exchange per register pair (kswap).
//   online softmax per row in fp32 (exp2 with scale*log2(e) folded in).
//   O^T[d][row] += V^T[d][tok] P^T[tok][row]  16x16x32 bf16 MFMA.  V moves
//       HBM -> LDS by direct (DMA) loads, never occupying VGPRs, and is read
//       back transposed with the LDS transpose read; P is split into two
//       bf16 parts (hi + lo, two MFMAs) so about 16 mantissa bits survive,
//       packed from the lane's own scores: the token order inside the QK
//       tile is permuted so each lane already holds the 8 consecutive tokens
//       its PV operand needs.
// HBM-bound: 64*d*2*2 bytes per block and row group; fp32 accumulate.
#include <limits.h>
#include <math.h>

#include "sda_attn_dev.hpp"
#include "sda_device.hpp"
#include "sda_internal.h"
#include "sda_ktilde_dev.hpp"
#include "sda_select_dev.hpp"

namespace sda {

// LDS of a workgroup of W waves: W V tiles, reused for the wave merge; the
// union lists of the grouped mode follow
// rows of the wave-merge area are padded by 4 floats: rows 16 apart in a wave's
// write land in different LDS banks
constexpr int kMergePad = 4;
__host__ __device__ inline size_t smem_base(int D, int RP, int W) {
    const size_t v = (size_t)W * kBlock * D * 2;
    const size_t m = (size_t)W * RP * (D + kMergePad + 2) * sizeof(float);
    return ((v > m ? v : m) + 15) / 16 * 16;
}
// LDS of the exact union: the C lists, the union ids and masks, per-wave
// counts
__host__ __device__ inline size_t union_extra(int C, int mode, int NB_cap, int n_sel_max, int W) {
    (void)NB_cap;
    if (C <= 1 || mode != 0) return 0;
    return ((size_t)C * n_sel_max * 3 * 4 + (size_t)W * 4 + 15) / 16 * 16;
}
constexpr int kMaxWaves = 10;

// list of blocks a workgroup walks, and which of the group's queries use each
struct ListView {
    const int32_t* gidx;   // global list (C == 1 or shared mode), or null
    const int32_t* gn;     // its entry count (global), read by the engine
    const int32_t* lidx;   // LDS list (exact union)
    const uint32_t* lmask; // LDS membership masks (exact union)
    int n;                 // entry count of the LDS list (or of the range)
    int lo;                // range list (NSA compressed and window branches): blocks lo .. lo + n - 1
    bool range;
};

// The buffer and token range one NSA branch attends to (three-branch mode only)
struct Branch {
    const uint16_t* kbase;  // key rows of this (b, g) in the branch's buffer
    const uint16_t* vbase;
    int row_cap;            // token rows in that buffer
    int lo_abs, hi_abs;     // valid tokens [lo_abs, hi_abs)
    int split_local;        // this workgroup's split inside the branch
    int n_split;            // the branch's splits
};

// Wait until at most N vector memory operations are outstanding; the K tile
// passes through as in-out operands so no use of it moves above the wait.
template <int N, int KS>
__device__ __forceinline__ void kwait(u32x4 (&kf)[4][KS]) {
    static_assert(KS == 2 || KS == 4, "head dim 64 or 128");
    if constexpr (KS == 4) {
        asm volatile("s_waitcnt vmcnt(%16)"
                     : "+v"(kf[0][0]), "+v"(kf[0][1]), "+v"(kf[0][2]), "+v"(kf[0][3]),
                       "+v"(kf[1][0]), "+v"(kf[1][1]), "+v"(kf[1][2]), "+v"(kf[1][3]),
                       "+v"(kf[2][0]), "+v"(kf[2][1]), "+v"(kf[2][2]), "+v"(kf[2][3]),
                       "+v"(kf[3][0]), "+v"(kf[3][1]), "+v"(kf[3][2]), "+v"(kf[3][3])
                     : "n"(N) : "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(%8)"
                     : "+v"(kf[0][0]), "+v"(kf[0][1]), "+v"(kf[1][0]), "+v"(kf[1][1]),
                       "+v"(kf[2][0]), "+v"(kf[2][1]), "+v"(kf[3][0]), "+v"(kf[3][1])
                     : "n"(N) : "memory");
    }
}

// Every vector load has landed; the Q fragments pass through as in-out operands
// so their registers stay reserved until here on every path (a wave whose
// list part is empty never reaches the K wait).
template <int NT, int KS>
__device__ __forceinline__ void qwait(u32x4 (&qf)[NT][KS]) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[nt][ks]));
}

// Merge the n_split partials (m, l, o) of one output row by log-sum-exp: one
// wave, lane owns columns lane + 64 i.  Partials are read in batches of
// kCombineMax with every load of a batch in flight at once, as agent-scope
// atomic loads (written moments ago by workgroups on other XCDs).
constexpr int kCombineMax = 8;
__device__ __forceinline__ float ld_part(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <int D, int RP>
__device__ __forceinline__ void merge_splits(const AttnArgs& a, int task, int r, int lane, int s_begin, int s_end,
                                             float& M, float& Ls, float (&Os)[D / kWave]) {
    constexpr int PER = D / kWave;
    const float* ml = a.part_ml + ((size_t)task * a.n_split * RP + r) * 2;
    const float* po = a.part_o + ((size_t)task * a.n_split * RP + r) * D + lane;
    M = -INFINITY;
    Ls = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) Os[i] = 0.f;
    for (int s0 = s_begin; s0 < s_end; s0 += kCombineMax) {
        float mv[kCombineMax], lv[kCombineMax], ov[kCombineMax][PER];
#pragma unroll
        for (int k = 0; k < kCombineMax; ++k) {
            const int s2 = s0 + k;
            const bool ok = s2 < s_end;
            mv[k] = ok ? ld_part(ml + (size_t)s2 * RP * 2) : -INFINITY;
            lv[k] = ok ? ld_part(ml + (size_t)s2 * RP * 2 + 1) : 0.f;
#pragma unroll
            for (int i = 0; i < PER; ++i) ov[k][i] = ok ? ld_part(po + (size_t)s2 * RP * D + i * kWave) : 0.f;
        }
        float Mn = M;
#pragma unroll
        for (int k = 0; k < kCombineMax; ++k) Mn = fmaxf(Mn, mv[k]);
        if (Mn == -INFINITY) continue;
        const float al = __builtin_amdgcn_exp2f(M - Mn);        // 0 on the first batch
        Ls *= al;
#pragma unroll
        for (int i = 0; i < PER; ++i) Os[i] *= al;
#pragma unroll
        for (int k = 0; k < kCombineMax; ++k) {
            const float sc = __builtin_amdgcn_exp2f(mv[k] - Mn);
            Ls += lv[k] * sc;
#pragma unroll
            for (int i = 0; i < PER; ++i) Os[i] += ov[k][i] * sc;
        }
        M = Mn;
    }
}

template <int D, int RP>
__device__ __forceinline__ void merge_row(const AttnArgs& a, int task, int r, size_t oi, int lane) {
    constexpr int PER = D / kWave;
    float M, Ls, Os[PER];
    merge_splits<D, RP>(a, task, r, lane, 0, a.n_split, M, Ls, Os);
#pragma unroll
    for (int i = 0; i < PER; ++i) a.out[oi * D + lane + i * kWave] = (Ls > 0.f) ? Os[i] / Ls : 0.f;
    if (lane == 0 && a.lse) a.lse[oi] = (Ls > 0.f) ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
}

// NSA gated sum ([SSV] NSA derivation step 6): each branch's splits merged by
// log-sum-exp and normalised, then o = g_c o_c + g_s o_s + g_w o_w; lse per
// branch (natural log, -inf for a branch with no token)
template <int D, int RP>
__device__ __forceinline__ void merge_row_nsa(const AttnArgs& a, int task, int r, size_t oi, int lane) {
    constexpr int PER = D / kWave;
    const int bounds[4] = {0, a.ns_c, a.ns_c + a.ns_s, a.n_split};
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
#pragma unroll
    for (int bi = 0; bi < 3; ++bi) {
        float M, Ls, Os[PER];
        merge_splits<D, RP>(a, task, r, lane, bounds[bi], bounds[bi + 1], M, Ls, Os);
        const float w = (Ls > 0.f) ? a.gates[oi * 3 + bi] / Ls : 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += Os[i] * w;
        if (lane == 0 && a.lse) a.lse[oi * 3 + bi] = (Ls > 0.f) ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) a.out[oi * D + lane + i * kWave] = acc[i];
}

// The same gated sum for two rows at once (rr[1] < 0: one row) when the row
// group has at most kCombineMax splits: every split of both rows (the three
// branches' splits are consecutive) and their gates in one batch of loads,
// then each branch merged from registers, in the same order as above.
template <int D, int RP>
__device__ __forceinline__ void merge_rows_nsa2(const AttnArgs& a, int task, const int (&rr)[2],
                                                const size_t (&oi)[2], int lane) {
    constexpr int PER = D / kWave;
    const int bounds[4] = {0, a.ns_c, a.ns_c + a.ns_s, a.n_split};
    float mv[2][kCombineMax], lv[2][kCombineMax], ov[2][kCombineMax][PER], gt[2][3];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = rr[q] < 0 ? rr[0] : rr[q];
        const float* ml = a.part_ml + ((size_t)task * a.n_split * RP + r) * 2;
        const float* po = a.part_o + ((size_t)task * a.n_split * RP + r) * D + lane;
#pragma unroll
        for (int k = 0; k < kCombineMax; ++k) {
            const bool ok = k < a.n_split;
            mv[q][k] = ok ? ld_part(ml + (size_t)k * RP * 2) : -INFINITY;
            lv[q][k] = ok ? ld_part(ml + (size_t)k * RP * 2 + 1) : 0.f;
#pragma unroll
            for (int i = 0; i < PER; ++i) ov[q][k][i] = ok ? ld_part(po + (size_t)k * RP * D + i * kWave) : 0.f;
        }
        const size_t o3 = (rr[q] < 0 ? oi[0] : oi[q]) * 3;
#pragma unroll
        for (int bi = 0; bi < 3; ++bi) gt[q][bi] = a.gates[o3 + bi];
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (rr[q] < 0) continue;                                 // wave-uniform
        float acc[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = 0.f;
#pragma unroll
        for (int bi = 0; bi < 3; ++bi) {
            float M = -INFINITY, Ls = 0.f, Os[PER];
#pragma unroll
            for (int i = 0; i < PER; ++i) Os[i] = 0.f;
#pragma unroll
            for (int k = 0; k < kCombineMax; ++k)
                if (k >= bounds[bi] && k < bounds[bi + 1]) M = fmaxf(M, mv[q][k]);
            if (M != -INFINITY) {
#pragma unroll
                for (int k = 0; k < kCombineMax; ++k)
                    if (k >= bounds[bi] && k < bounds[bi + 1]) {
                        const float sc = __builtin_amdgcn_exp2f(mv[q][k] - M);   // 0 for an empty split
                        Ls += lv[q][k] * sc;
#pragma unroll
                        for (int i = 0; i < PER; ++i) Os[i] += ov[q][k][i] * sc;
                    }
            }
            const float w = (Ls > 0.f) ? gt[q][bi] / Ls : 0.f;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] += Os[i] * w;
            if (lane == 0 && a.lse)
                a.lse[oi[q] * 3 + bi] = (Ls > 0.f) ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) a.out[oi[q] * D + lane + i * kWave] = acc[i];
    }
}

// ---- decode step: the next layer's scoring and selection ------------------------
// Workgroup w scores chunks w * per_wg + i (i < per_wg, one per group of four
// waves) of the next layer's compressed keys against its indexer vectors,
// keeps each chunk's top-k keys (level 1), and the last workgroup to finish a
// row's chunks merges them into the row's block set (level 2).  Loads,
// arithmetic and merges are the scoring launch's, so the block sets equal
// sda_score_select's bit for bit.  LDS at `sl` (step_lds_bytes): per group the
// chunk's scores and four wave lists, then the level-2 buffers and flags.
// These workgroups follow the attention grid: the dispatcher starts them on
// the compute units the attention workgroups leave, so their loads fill the
// memory pipe while the attention's split merges and stragglers finish.
struct StepPos {
    int grp, t, row, ch, nb;
    bool has;
};

__device__ __forceinline__ StepPos step_pos(const AttnArgs& a, int w) {
    const StepScore& st = a.step;
    StepPos p;
    p.grp = threadIdx.x / kChunk;
    p.t = threadIdx.x % kChunk;
    const int cid = w * st.per_wg + p.grp;
    p.has = p.grp < st.per_wg && cid < st.sel.rows * st.cpr;
    p.row = p.has ? cid / st.cpr : 0;
    p.ch = p.has ? cid - p.row * st.cpr : 0;
    p.nb = min((ld_ro(st.sel.seq_len + p.row / st.sel.H_kv) + kBlock - 1) / kBlock, st.sel.NB_cap);
    return p;
}

__device__ __forceinline__ char* step_group_lds(const AttnArgs& a, const StepPos& p, char* sl) {
    return sl + (size_t)min(p.grp, a.step.per_wg - 1) * step_group_lds_bytes(a.step.sel.top_k);
}

// scores of this group's chunk into LDS (no barrier)
template <int D>
__device__ __forceinline__ void step_scores(const AttnArgs& a, const StepPos& p, char* sl) {
    constexpr int EPL = D / 16;                 // bf16 elements per lane of one pooled key (16 lanes per key)
    constexpr int STEPS = kChunk / 16;          // 16 blocks per group step, all in flight at once
    using KLoad = typename std::conditional<EPL == 8, u32x4, u32x2>::type;
    const StepScore& st = a.step;
    const int j0 = p.ch * kChunk;
    if (!p.has || j0 >= p.nb) return;
    const int lane = p.t % kWave, wave = p.t / kWave, li = lane & 15;
    float* sc = reinterpret_cast<float*>(step_group_lds(a, p, sl));
    const KLoad fw = *reinterpret_cast<const KLoad*>(st.vec + (size_t)p.row * D + li * EPL);
    const uint16_t* ktr = st.kt + (size_t)p.row * st.sel.NB_cap * D + li * EPL;
    KLoad kv[STEPS];
    int jj[STEPS];
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
        jj[u] = j0 + u * 16 + wave * 4 + (lane >> 4);
        // past the length: re-read the last block (cached), result unused
        kv[u] = __builtin_nontemporal_load(reinterpret_cast<const KLoad*>(ktr + (size_t)min(jj[u], p.nb - 1) * D));
    }
    float fv[EPL];
    const uint32_t* wp = reinterpret_cast<const uint32_t*>(&fw);
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) {
        fv[2 * i] = bf16lo(wp[i]);
        fv[2 * i + 1] = bf16hi(wp[i]);
    }
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
        const float s = key_dot<EPL>(fv, reinterpret_cast<const uint32_t*>(&kv[u]));
        if (li == 0 && jj[u] < p.nb) sc[jj[u] - j0] = s;
    }
}

// level 1 of this group's chunk (every thread of the workgroup calls it)
__device__ __forceinline__ void step_level1(const AttnArgs& a, const StepPos& p, char* sl) {
    const StepScore& st = a.step;
    const int lo = min(st.sel.n_init, p.nb);    // candidates are [lo, hi)
    const int hi = max(lo, p.nb - st.sel.n_local);
    char* gl = step_group_lds(a, p, sl);
    __syncthreads();                            // scores complete
    chunk_top_k(reinterpret_cast<const float*>(gl), p.ch * kChunk, lo, hi, st.sel.top_k, p.has,
                reinterpret_cast<uint64_t*>(gl + kChunk * 4), st.cand + ((size_t)p.row * st.cpr + p.ch) * st.sel.top_k,
                p.t);
}

// arrival per chunk and level 2 in the last workgroup of each row (every
// thread of the workgroup calls it; it drains this workgroup's stores)
__device__ __forceinline__ void step_finish(const AttnArgs& a, const StepPos& p, int w, char* sl) {
    const StepScore& st = a.step;
    const SelectArgs& sel = st.sel;
    const int K = sel.top_k;
    const int P = pow2_at_least(K);
    uint64_t* fA = reinterpret_cast<uint64_t*>(sl + (size_t)st.per_wg * step_group_lds_bytes(K));
    uint64_t* fB = fA + (size_t)P * st.cpr;
    int* last = reinterpret_cast<int*>(fB + (size_t)P * ((st.cpr + 1) / 2));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // this wave's list stores have completed
    __syncthreads();
    if (p.t == 0 && p.grp < st.per_wg) {
        last[p.grp] = p.has && arrive(st.counters + p.row) == st.cpr - 1;
        if (last[p.grp]) acquire_agent();
    }
    __syncthreads();
    for (int g2 = 0; g2 < st.per_wg; ++g2) {
        if (!last[g2]) continue;                            // uniform: one LDS flag
        const int r2 = (w * st.per_wg + g2) / st.cpr;
        const int nb2 = min((ld_ro(sel.seq_len + r2 / sel.H_kv) + kBlock - 1) / kBlock, sel.NB_cap);
        finish_row<true>(sel, st.cand + (size_t)r2 * st.cpr * K, st.cpr, r2, nb2, fA, fB);
        if (threadIdx.x == 0) __hip_atomic_store(st.counters + r2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();                                        // LDS free again
}

// a workgroup that only scores and selects: `passes` rounds of per_wg chunks
template <int D>
__device__ __forceinline__ void step_score_role(const AttnArgs& a, int w, char* smem) {
    for (int pass = 0; pass < a.step.passes; ++pass) {
        const int vw = w * a.step.passes + pass;
        const StepPos p = step_pos(a, vw);
        step_scores<D>(a, p, smem);
        step_level1(a, p, smem);
        step_finish(a, p, vw, smem);
    }
}

// The refresh of this layer's compressed keys ([SparDA] §4.2 step 1: the key
// just appended updates its block's mean): the blocks touched by the tokens
// [ref_len_old, seq_len) of each row, recomputed whole with the arithmetic of
// sda_update_compressed_keys.  Item i = (row, i-th touched block).
template <int D>
__device__ __forceinline__ bool refresh_item(const AttnArgs& a, int item, int& row, int& j, int& t0, int& n) {
    const StepScore& st = a.step;
    row = item / st.ref_blocks;                         // b * H_kv + g
    if (row >= a.B * a.H_kv) return false;
    const int b = row / a.H_kv;
    const int lo = max(ld_ro(st.ref_len_old + b), 0);
    const int hi = min(ld_ro(a.seq_len + b), a.T_cap);
    if (hi <= lo) return false;
    j = lo / kBlock + (item - row * st.ref_blocks);
    if (j > (hi - 1) / kBlock || j >= st.ref_NB_cap) return false;
    t0 = j * kBlock;
    n = min(kBlock, hi - t0);
    return true;
}

// by a workgroup of its own, placed after the scoring workgroups: item w, all
// threads (one barrier).  Measured at the 128K workload: +0.3 us per step
// launch (+0.9 us per step of the 80-step graph), against 3.4 us for a
// separate refresh launch; refresh workgroups dispatched before the scoring
// ones, or the scoring workgroups' idle waves doing the refresh, were slower
// (+1.8 and +2.1 us per step launch)
template <int D>
__device__ __forceinline__ void step_refresh_role(const AttnArgs& a, int w, char* smem) {
    int row, j, t0, n;
    if (!refresh_item<D>(a, w, row, j, t0, n)) return;       // uniform over the workgroup
    ktilde_window<D>(a.k, a.step.ref_kt, row, j, t0, n, a.T_cap, a.step.ref_NB_cap, threadIdx.x,
                     reinterpret_cast<double (*)[D + 2]>(smem));
}

// KSTREAM: the K loads carry the non-temporal hint and the V direct loads the
// default policy (the decode launch alone); otherwise the other way round (the
// decode inside the step launch, where the scoring workgroups stream K~ beside
// it: 24.1 against 26.8 us per step at the 128K workload).
// NSA: the three-branch mode; `br` gives this workgroup's branch buffer,
// token range and split inside the branch (unused otherwise).
template <int D, int NT, bool KSTREAM, bool NSA = false>
__device__ __forceinline__ void run_tile_engine(const AttnArgs& a, ListView L, int b, int g, int q0,
                                                int Cg, int split, int task, char* smem, const Branch& br = Branch{}) {
    constexpr int KS = D / 32;            // QK k-steps
    constexpr int MTD = D / 16;           // PV m-tiles over d
    constexpr int RP = NT * 16;           // padded rows
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
    const int W = blockDim.x / kWave;     // waves per workgroup (one block each, normally)
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int G = a.G;
    const int R = Cg * G;
    // The wave's block ids (global list) arrive by one vector load, lane k
    // holding its k-th entry; the length and the list count are scalar reads
    // issued beside it, then the Q loads; nothing waits for any of them until
    // all are issued, so the first K/V loads follow one round trip.
    const bool glist = L.gidx != nullptr;
    const int n_range = glist ? a.n_sel_max : L.n;
    const int s_loc = NSA ? br.split_local : split;
    const int ns_b = NSA ? br.n_split : a.n_split;
    const int e_begin = (s_loc * n_range) / ns_b;
    const int e_end = ((s_loc + 1) * n_range) / ns_b;
    const int32_t* slot_row = (a.slot && glist) ? a.slot + (L.gidx - a.block_idx) : nullptr;
    int e = e_begin + wave;
    int T = ld_ro(a.seq_len + b);
    int n_g = ld_ro(glist ? L.gn : a.seq_len + b);        // unused without a global list
    int id_v = -1, slot_v = -1;            // entries e + (it + lane) * W, it = 0, 64, ...
    auto load_ids = [&](int e0) {
        const int ee = e0 + lane * W;
        const bool ok = ee < e_end;
        id_v = ok ? L.gidx[ee] : -1;
        if (slot_row) slot_v = ok ? slot_row[ee] : -1;
    };
    if (glist) load_ids(e);

    // Q fragments (B operand of S^T = K Q^T): row nt*16 + li, d = ks*32 + lg*8
    u32x4 qf[NT][KS];
    int rowq[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + li;
        const int c = r / G, h = r - c * G;
        rowq[nt] = c;
        const uint16_t* qp = a.q + (((size_t)b * a.NQ + q0 + min(c, Cg - 1)) * a.H_q + (size_t)g * G + h) * D + lg * 8;
        // padding rows (r >= R) read a real row; their columns are never written back.
        // Issued as asm like the K loads: the first K wait covers them.
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(qf[nt][ks]) : "v"(qp + ks * 32) : "memory");
    }
    // the scalar reads are first used here, after every load above is issued
    asm volatile("" : "+s"(T), "+s"(n_g));
    if (glist) L.n = min(max(n_g, 0), a.n_sel_max);
    const int hi_abs = NSA ? br.hi_abs : T;            // valid tokens end here
    const int row_cap = NSA ? br.row_cap : a.T_cap;     // token rows of the buffer
    const int nb = (hi_abs + kBlock - 1) / kBlock;
    const int blocks_cap = (row_cap + kBlock - 1) / kBlock;


    floatx4 o[MTD][NT];
#pragma unroll
    for (int i = 0; i < MTD; ++i)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[i][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run[NT], l_run[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.f;
    }

    char* vs = smem + (size_t)wave * VTile<D>::kBytes;
    SDA_LDS char* vs_lds = (SDA_LDS char*)(vs);
    const uint16_t* kv_k = NSA ? br.kbase : a.k + ((size_t)b * a.H_kv + g) * a.T_cap * D;
    const uint16_t* kv_v = NSA ? br.vbase : a.v + ((size_t)b * a.H_kv + g) * a.T_cap * D;
    // global lists are split over their static width, so a wave's first block
    // id is read together with the row's entry count; entries past the count
    // are padding and skipped

    // V direct loads: LDS slot (i, lane) holds row i*VRPI + lane/VLPR, 16-byte piece
    // lane % VLPR of the permuted row; the lane fetches the matching logical piece
    constexpr int VLPR = VTile<D>::kRowBytes / 16;         // lanes per V row
    constexpr int VRPI = kWave / VLPR;                      // V rows per direct load
    const int v_lrow = lane / VLPR;
    const int v_rb = (lane % VLPR) * 16;
    const int tr_col = (li & 3) * 8;       // bytes inside the 32-byte chunk for the transposed reads

    for (int it = 0; e < e_end; e += W, ++it) {
        int j, phys;
        uint32_t memb;
        if (glist) {
            if (it && (it & (kWave - 1)) == 0) load_ids(e);
            j = __builtin_amdgcn_readlane(id_v, it & (kWave - 1));
            phys = slot_row ? __builtin_amdgcn_readlane(slot_v, it & (kWave - 1)) : j;
            memb = 0xffffffffu;
        } else if (NSA && L.range) {
            j = L.lo + e;
            phys = j;
            memb = 0xffffffffu;
        } else {
            j = L.lidx[e];
            phys = j;
            memb = L.lmask[e];
        }
        if (e >= L.n) break;
        if (j < 0 || j >= nb || phys < 0 || phys >= blocks_cap) continue;
        const int nvalid = min(kBlock, hi_abs - j * kBlock);
        if (phys * kBlock + nvalid > row_cap) continue;
        const int tfirst = NSA ? max(0, br.lo_abs - j * kBlock) : 0;   // first valid token of the block
        const char* kb = reinterpret_cast<const char*>(kv_k + (size_t)phys * kBlock * D);
        const char* vb = reinterpret_cast<const char*>(kv_v + (size_t)phys * kBlock * D);
        const int tmax = nvalid - 1;
        const bool full = (nvalid == kBlock) && (memb == 0xffffffffu) && tfirst == 0;   // wave-uniform

        // ---- K into registers (MFMA A layout), then V into LDS by direct loads;
        //      everything is in flight before the first wait, and QK and the
        //      softmax wait only for K (V is still on its way) --------------------------
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // previous tile's LDS reads are done
        // K loads are issued as asm so that the compiler does not fold the V
        // direct loads issued after them into its wait for K: the explicit
        // vmcnt wait below lets exactly the kLoads V loads stay in flight.
        // Each load covers whole 128-byte lines: load (mt, h, x) brings rows
        // tok_of(mt, 8x + l%8) x bytes [128h, 128h + 128) (see kswap).
        u32x4 kf[4][KS];
        const uint32_t kline = (uint32_t)(((lane >> 4) + 4 * ((lane >> 3) & 1)) * 16);   // piece inside a line
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const uint32_t off = (uint32_t)min(tok_of(mt, 8 * x + (lane & 7)), tmax) * (D * 2) + kline;
#pragma unroll
                for (int h = 0; h < KS / 2; ++h)
                    if constexpr (KSTREAM)
                        asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(kf[mt][2 * h + x]) : "v"(kb + off + h * 128) : "memory");
                    else
                        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(kf[mt][2 * h + x]) : "v"(kb + off + h * 128) : "memory");
            }
#pragma unroll
        for (int i = 0; i < VTile<D>::kLoads; ++i) {
            const int t = i * VRPI + v_lrow;
            const uint32_t off = (uint32_t)min(t, tmax) * VTile<D>::kRowBytes +
                                 (uint32_t)(v_rb ^ (VTile<D>::perm(t) << 5));
            lds_dma16<KSTREAM ? 0 : 2>(vb + off, vs_lds + i * kWave * 16);   // 2: non-temporal
        }
        kwait<VTile<D>::kLoads, KS>(kf);                    // K (and everything before it) has landed
        kswap<KS>(kf);
        if (it == 0) {                                       // so have the Q fragments
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[nt][ks]));
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- S^T = K Q^T ----------------------------------------------------------
        floatx4 s[4][NT];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(kf[mt][ks], qf[nt][ks], acc);
                s[mt][nt] = acc;
            }

        // ---- online softmax per row (log2 domain; the scale is folded into the exponent)
        u32x4 pf[NT][2], pl[NT][2];
        const float c = a.scale_log2;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (!full) {
                const bool live = (memb >> rowq[nt]) & 1u;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!(live && tok_of(mt, lg * 4 + i) < nvalid && tok_of(mt, lg * 4 + i) >= tfirst))
                            s[mt][nt][i] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                mx = fmaxf(mx, fmaxf(fmaxf(s[mt][nt][0], s[mt][nt][1]), fmaxf(s[mt][nt][2], s[mt][nt][3])));
            mx = cross4_max(mx) * c;                            // raw max, scaled (c > 0)
            const float m_new = fmaxf(m_run[nt], mx);
            const bool any = m_new != -INFINITY;
            const float m_use = any ? m_new : 0.f;
            float psum = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[mt][nt][i], c, -m_use));   // exp2(-inf) = 0
                    s[mt][nt][i] = p;
                    psum += p;
                }
            psum = cross4_sum(psum);
            if (m_run[nt] != -INFINITY) {                       // earlier blocks of this wave: rescale
                const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
                l_run[nt] *= alpha;
#pragma unroll
                for (int i = 0; i < MTD; ++i) {
                    o[i][nt][0] *= alpha;
                    o[i][nt][1] *= alpha;
                    o[i][nt][2] *= alpha;
                    o[i][nt][3] *= alpha;
                }
            }
            l_run[nt] += psum;
            m_run[nt] = m_new;
            // P^T B operand for token half kh: slot jj = (mt&1)*4 + i with mt = 2*kh + (jj>>2);
            // P = hi + lo, both bf16 (hardware round-to-nearest-even packs)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float p0 = s[2 * kh + (w >> 1)][nt][(w & 1) * 2];
                    const float p1 = s[2 * kh + (w >> 1)][nt][(w & 1) * 2 + 1];
                    const bf16x2 h = {(__bf16)p0, (__bf16)p1};
                    const bf16x2 r = {(__bf16)(p0 - (float)h[0]), (__bf16)(p1 - (float)h[1])};
                    pf[nt][kh][w] = __builtin_bit_cast(uint32_t, h);
                    pl[nt][kh][w] = __builtin_bit_cast(uint32_t, r);
                }
        }

        // ---- O^T += V^T P^T (V^T by LDS transpose reads) ------------------------------
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // the direct loads have landed
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int md = 0; md < MTD; ++md) {
                u32x4 va;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int t = kh * 32 + lg * 8 + hh * 4 + (li >> 2);
                    const int pc = md ^ VTile<D>::perm(t);
                    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (SDA_LDS v4i16*)(vs_lds + t * VTile<D>::kRowBytes + (pc << 5) + tr_col));
                    const uint2 rr = __builtin_bit_cast(uint2, r);
                    va[2 * hh] = rr.x;
                    va[2 * hh + 1] = rr.y;
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    o[md][nt] = mfma16x16x32(va, pf[nt][kh], o[md][nt]);
                    o[md][nt] = mfma16x16x32(va, pl[nt][kh], o[md][nt]);
                }
            }
        }
    }

    qwait<NT, KS>(qf);

    // ---- merge the waves of this workgroup through LDS -------------------------------
    // Each wave publishes (m, l) per row and its o; after one barrier a thread
    // owns four consecutive columns of one row and reads every wave's values
    // in one unrolled batch (no dependent LDS round trips).
    __syncthreads();
    float* sm_m = reinterpret_cast<float*>(smem);        // [W][RP]
    float* sm_l = sm_m + W * RP;                          // [W][RP]
    float* sm_o = sm_l + W * RP;                          // [W][RP][D + kMergePad]
    constexpr int OS = D + kMergePad;                     // row stride of sm_o
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + li;
        if (lg == 0) {
            sm_m[wave * RP + r] = m_run[nt];
            sm_l[wave * RP + r] = l_run[nt];
        }
#pragma unroll
        for (int md = 0; md < MTD; ++md)
            *reinterpret_cast<floatx4*>(&sm_o[(wave * RP + r) * OS + md * 16 + lg * 4]) = o[md][nt];
    }
    __syncthreads();

    const bool final_out = (a.n_split == 1);
    constexpr int QPR = D / 4;                            // column quads per row
    for (int qi = threadIdx.x; qi < R * QPR; qi += blockDim.x) {
        const int r = qi / QPR, d4 = (qi - r * QPR) * 4;
        float mw[kMaxWaves], lw[kMaxWaves];
        floatx4 ow[kMaxWaves];
#pragma unroll
        for (int w = 0; w < kMaxWaves; ++w) {
            if (w < W) {
                mw[w] = sm_m[w * RP + r];
                lw[w] = sm_l[w * RP + r];
                ow[w] = *reinterpret_cast<const floatx4*>(&sm_o[(w * RP + r) * OS + d4]);
            } else {
                mw[w] = -INFINITY;
                lw[w] = 0.f;
                ow[w] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kMaxWaves; ++w) M = fmaxf(M, mw[w]);
        float Ls = 0.f;
        floatx4 Os = floatx4{0.f, 0.f, 0.f, 0.f};
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kMaxWaves; ++w) {
                const float sc = __builtin_amdgcn_exp2f(mw[w] - M);      // 0 for absent waves
                Ls += lw[w] * sc;
                Os[0] += ow[w][0] * sc;
                Os[1] += ow[w][1] * sc;
                Os[2] += ow[w][2] * sc;
                Os[3] += ow[w][3] * sc;
            }
        }
        if (final_out) {
            const int c = r / G, h = r - (r / G) * G;
            const size_t oi = ((size_t)b * a.NQ + q0 + c) * a.H_q + (size_t)g * G + h;
            const float inv = (Ls > 0.f) ? 1.f / Ls : 0.f;
            *reinterpret_cast<floatx4*>(&a.out[oi * D + d4]) =
                floatx4{Os[0] * inv, Os[1] * inv, Os[2] * inv, Os[3] * inv};
            if (d4 == 0 && a.lse) a.lse[oi] = (Ls > 0.f) ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
        } else {
            const size_t pi = ((size_t)task * a.n_split + split) * RP + r;
            // device-scope (write-through) stores: the merging workgroup may
            // sit on another XCD; the four columns go out as one 16-byte
            // store from the split's wave-uniform base
            st_agent16(a.part_o + ((size_t)task * a.n_split + split) * RP * D, (uint32_t)((r * D + d4) * 4), Os);
            if (d4 == 0)
                __hip_atomic_store(reinterpret_cast<uint64_t*>(&a.part_ml[pi * 2]),
                                   ((uint64_t)__float_as_uint(Ls) << 32) | __float_as_uint(M),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (final_out) return;

    // ---- the last workgroup of this row group merges the splits ----------------------
    // Every wave waits for its partial stores to complete; after a barrier one
    // agent-scope increment per workgroup tells the last arrival, which then
    // acquires, that every split is readable (arrive()).
    int* last = reinterpret_cast<int*>(smem);           // the merge area is free again
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        *last = arrive(&a.counters[task]) == a.n_split - 1;
        if (*last) acquire_agent();
    }
    __syncthreads();
    if (!*last) return;
    auto out_row = [&](int r) { return ((size_t)b * a.NQ + q0 + r / G) * a.H_q + (size_t)g * G + (r - (r / G) * G); };
    if (NSA && a.n_split <= kCombineMax) {
        // two rows per wave at a time, all their loads in flight together
        for (int r = wave; r < R; r += 2 * W) {
            const int rr[2] = {r, r + W < R ? r + W : -1};
            const size_t oi[2] = {out_row(r), rr[1] >= 0 ? out_row(rr[1]) : 0};
            if constexpr (NSA) merge_rows_nsa2<D, RP>(a, task, rr, oi, lane);
        }
    } else {
        for (int r = wave; r < R; r += W) {
            if constexpr (NSA) merge_row_nsa<D, RP>(a, task, r, out_row(r), lane);
            else merge_row<D, RP>(a, task, r, out_row(r), lane);
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&a.counters[task], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// STEP: the decode step; workgroups past the attention grid score and select
// (the dispatcher starts them as attention workgroups retire).
// NSA: the three-branch mode; split x of a row group serves the compressed
// branch (x < ns_c), the listed blocks (x < ns_c + ns_s) or the window.
// REF (with STEP): ref_rows grid rows of workgroups after the scoring ones
// refresh the decoded layer's compressed keys (a variant of its own, so the
// step without it keeps its code).
template <int D, int NT, bool STEP, bool NSA = false, bool REF = false>
__global__ __launch_bounds__(NT == 1 ? kMaxWaves * 64 : 256) void attn_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    if constexpr (STEP) {
        const int attn_rows = a.B * a.n_groups * a.H_kv;
        if ((int)blockIdx.y >= attn_rows) {
            const int w = ((int)blockIdx.y - attn_rows) * (int)gridDim.x + (int)blockIdx.x;
            if constexpr (REF) {
                const int score_wgs = ((int)gridDim.y - attn_rows - a.step.ref_rows) * (int)gridDim.x;
                if (w >= score_wgs) {
                    step_refresh_role<D>(a, w - score_wgs, smem);
                    return;
                }
            }
            step_score_role<D>(a, w, smem);
            return;
        }
    }
    const int task = a.task0 + (int)blockIdx.y;
    const int split = blockIdx.x;
    const int g = task % a.H_kv;
    const int t2 = task / a.H_kv;
    const int grp = t2 % a.n_groups;
    const int b = t2 / a.n_groups;
    const int q0 = grp * a.C;
    const int Cg = min(a.C, a.NQ - q0);

    ListView L{};
    Branch br{};
    int branch = 1;                                  // NSA: 0 compressed, 1 listed blocks, 2 window
    if constexpr (NSA) {
        branch = split < a.ns_c ? 0 : (split < a.ns_c + a.ns_s ? 1 : 2);
        const int T = ld_ro(a.seq_len + b);
        const size_t kvrow = (size_t)b * a.H_kv + g;
        if (branch == 0) {                           // every compressed entry present at length T
            const int ncmp = min((T + a.cmp_stride - 1) / a.cmp_stride, a.NC_cap);
            br = Branch{a.kc + kvrow * a.NC_cap * D, a.vc + kvrow * a.NC_cap * D, a.NC_cap, 0, ncmp, split, a.ns_c};
            L.range = true;
            L.lo = 0;
            L.n = (ncmp + kBlock - 1) / kBlock;
        } else {                                     // the cache: listed blocks, or tokens [T - window, T)
            const int lo = branch == 2 ? max(0, T - a.window) : 0;
            const int s0 = branch == 2 ? a.ns_c + a.ns_s : a.ns_c;
            br = Branch{a.k + kvrow * a.T_cap * D, a.v + kvrow * a.T_cap * D, a.T_cap, lo, T, split - s0,
                        branch == 2 ? a.n_split - s0 : a.ns_s};
            if (branch == 2) {
                L.range = true;
                L.lo = lo / kBlock;
                L.n = T > lo ? (T - 1) / kBlock - lo / kBlock + 1 : 0;
            }
        }
    }
    char* after_v = smem + smem_base(D, NT * 16, blockDim.x / kWave);
    const size_t row0 = ((size_t)b * a.NQ + q0) * a.H_kv + g;   // block_idx row of the group's first query
    if (NSA && branch != 1) {
        // range list set above
    } else if (a.C == 1 || a.mode == 1) {
        L.gidx = a.block_idx + row0 * a.n_sel_max;
        L.gn = a.n_sel + row0;
    } else {
        // exact union of the group's ascending lists: entry (c, e) joins the
        // union unless an earlier query of the group, or the entry before it,
        // lists the same block; its membership mask comes from a binary
        // search in every list.  Joining entries are compacted in (c, e) order.
        // (the global-list path reads the length inside the engine, after its
        // block-id load is on its way: no round trip before that load)
        const int nb = (ld_ro(a.seq_len + b) + kBlock - 1) / kBlock;
        const int nsm = a.n_sel_max;
        const int W = blockDim.x / kWave;
        int32_t* lst = reinterpret_cast<int32_t*>(after_v);                          // [C][nsm]
        int32_t* lidx = lst + (size_t)a.C * nsm;                                     // [C * nsm]
        uint32_t* lmask = reinterpret_cast<uint32_t*>(lidx + (size_t)a.C * nsm);     // [C * nsm]
        int* wtot = reinterpret_cast<int*>(lmask + (size_t)a.C * nsm);              // [W]
        const int n_ent = Cg * nsm;
        for (int i = threadIdx.x; i < n_ent; i += blockDim.x) {
            const int c = i / nsm, e = i - (i / nsm) * nsm;
            const size_t rc = row0 + (size_t)c * a.H_kv;
            const int n_c = min(max(a.n_sel[rc], 0), nsm);
            int j = (e < n_c) ? a.block_idx[rc * nsm + e] : INT_MAX;   // past the count: sorts last
            if (j < 0 || j >= nb || j >= a.NB_cap) j = INT_MAX;
            lst[i] = j;
        }
        __syncthreads();
        auto contains = [&](int c, int v) {
            const int32_t* Lc = lst + c * nsm;
            int lo = 0, hi = nsm;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (Lc[mid] < v) lo = mid + 1;
                else hi = mid;
            }
            return lo < nsm && Lc[lo] == v;
        };
        const int lane = __lane_id(), wv = threadIdx.x / kWave;
        int base = 0;
        for (int i0 = 0; i0 < n_ent; i0 += blockDim.x) {
            const int i = i0 + threadIdx.x;
            bool first = false;
            uint32_t mk = 0;
            int v = INT_MAX;
            if (i < n_ent) {
                const int c = i / nsm, e = i - (i / nsm) * nsm;
                v = lst[i];
                first = v != INT_MAX && !(e > 0 && lst[i - 1] == v);
                for (int c2 = 0; c2 < c && first; ++c2) first = !contains(c2, v);
                if (first)
                    for (int c2 = 0; c2 < Cg; ++c2) mk |= (uint32_t)contains(c2, v) << c2;
            }
            const uint64_t bal = __ballot(first);
            if (lane == 0) wtot[wv] = __popcll(bal);
            __syncthreads();
            int off = base, tot = 0;
            for (int w2 = 0; w2 < W; ++w2) {
                off += (w2 < wv) ? wtot[w2] : 0;
                tot += wtot[w2];
            }
            if (first) {
                const int pos = off + __popcll(bal & ((1ull << lane) - 1ull));
                lidx[pos] = v;
                lmask[pos] = mk;
            }
            base += tot;
            __syncthreads();                                   // wtot is rewritten by the next chunk
        }
        L.lidx = lidx;
        L.lmask = lmask;
        L.n = base;
    }
    run_tile_engine<D, NT, !STEP, NSA>(a, L, b, g, q0, Cg, split, task, smem, br);
    // written last: no global store precedes the engine's loads, so the
    // compiler may read lists and lengths through the scalar cache
    if (a.union_count && a.C > 1 && split == (NSA ? a.ns_c : 0) && threadIdx.x == 0)
        a.union_count[((size_t)b * a.n_groups + grp) * a.H_kv + g] =
            L.gidx ? min(max(ld_ro(L.gn), 0), a.n_sel_max) : L.n;
}

int attn_rows_pad(int C, int G) { return (C * G <= 16) ? 16 : 32; }

constexpr size_t kLdsPerCU = 160 * 1024;
constexpr int kPlanMaxSplits = 1024;          // the planner tries at most this many splits
constexpr int kMaxGridRows = 65535;


// Workgroups of one shape that a compute unit holds at once: its LDS share,
// and the wave slots of its four SIMDs (slots_simd waves each at the engine's
// register count).  Workgroups of up to four waves pack over the SIMDs; a
// larger one takes ceil(W / 4) slots on every SIMD (measured on gfx950 with
// workgroups that hold their compute unit: at 150-168 VGPRs, three waves per
// SIMD, five- to ten-wave workgroups run one per compute unit, four-wave ones
// three, two-wave ones six).
static int wgs_per_cu(int W, size_t lds, int slots_simd) {
    const int by_lds = (int)(kLdsPerCU / lds);
    const int by_slots = W <= 4 ? (4 * slots_simd) / W : slots_simd / ((W + 3) / 4);
    return max(1, min(by_lds, by_slots));
}

// Launch shape of the attention kernel: W waves per workgroup, n_split
// workgroups per row group; a wave walks its split's entries W apart, so it
// handles ceil(list / (n_split * W)) blocks one after another.  Cost of a
// shape = dispatch rounds x (kRoundCost + blocks per wave): a round's head
// (launch, block ids, first K) and tail (merges) cost about two blocks' time
// (at the 64K verification workload, 19 blocks per row: one round of
// four-wave workgroups, five blocks per wave, 29.2 us; two rounds of
// ten-wave ones, two blocks per wave, 34.2 us; two rounds of five-wave
// ones 32.2 us).  Workgroups take at least four waves (or the split's whole
// share): single-wave workgroups of many splits measured slower still (42.5
// us there).  Among the cheapest, keep the one with the most blocks in
// flight in the first round (at most all of them), then the one that
// reaches the most CUs, then the fewest splits (less partial traffic), then
// the fewest waves.
constexpr int kRoundCost = 2;
AttnPlan attn_plan(int d, int rows_pad, int tasks, int list_max, int C, int mode, int NB_cap, int n_sel_max,
                   int split_k) {
    const int max_w = rows_pad == 16 ? kMaxWaves : 4;
    const int slots_simd = rows_pad == 16 ? 3 : 1;     // resident waves per SIMD (168 or 356 VGPRs)
    if (list_max < 1) list_max = 1;
    if (split_k > 0) {
        int W = (list_max + split_k - 1) / split_k;
        if (W > max_w) W = max_w;
        if (W < 1) W = 1;
        while (W > 1 && smem_base(d, rows_pad, W) + union_extra(C, mode, NB_cap, n_sel_max, W) > kLdsPerCU)
            --W;                                           // fewer waves (each walks more blocks) to fit the LDS
        return AttnPlan{W, split_k};
    }
    AttnPlan best{1, 1};
    long long best_cost = -1, best_flight = -1, best_cus = -1;
    const long long total = (long long)tasks * list_max;
    for (int ns = 1; ns <= min(list_max, kPlanMaxSplits); ++ns) {
        const int per_split = (list_max + ns - 1) / ns;
        for (int W = min(4, per_split); W <= min(max_w, per_split); ++W) {
            const size_t lds = smem_base(d, rows_pad, W) + union_extra(C, mode, NB_cap, n_sel_max, W);
            if (lds > kLdsPerCU) continue;
            const int per_cu = wgs_per_cu(W, lds, slots_simd);
            const long long wgs = (long long)tasks * ns;
            const long long cap = (long long)kCUs * per_cu;
            const long long rounds = (wgs + cap - 1) / cap;
            const long long cost = rounds * (kRoundCost + (per_split + W - 1) / W);
            long long flight = (wgs < cap ? wgs : cap) * W;
            if (flight > total) flight = total;
            const long long cus = wgs < kCUs ? wgs : kCUs;
            if (best_cost < 0 || cost < best_cost ||
                (cost == best_cost && (flight > best_flight || (flight == best_flight && cus > best_cus)))) {
                best = AttnPlan{W, ns};
                best_cost = cost;
                best_flight = flight;
                best_cus = cus;
            }
        }
    }
    return best;
}

size_t attn_ws_bytes(int tasks, int n_split, int rows_pad, int d) {
    if (n_split <= 1) return 0;
    const size_t counters = ((size_t)tasks * sizeof(int) + 255) / 256 * 256;
    return counters + (size_t)tasks * n_split * rows_pad * ((size_t)d + 2) * sizeof(float);
}

size_t attn_smem_bytes_host(int d, int rows_pad, int W, int C, int mode, int NB_cap, int n_sel_max) {
    return smem_base(d, rows_pad, W) + union_extra(C, mode, NB_cap, n_sel_max, W);
}

template <int D, int NT>
static hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
    const int tasks = a.B * a.n_groups * a.H_kv;
    const bool step = a.step.cand != nullptr;
    size_t smem = attn_smem_bytes_host(D, NT * 16, a.waves, a.C, a.mode, a.NB_cap, a.n_sel_max);
    int extra_rows = 0;                        // grid rows of workgroups that only score or refresh
    AttnArgs aa = a;
    if (step) {
        size_t need = step_lds_bytes(a.step.sel.top_k, a.step.cpr, a.step.per_wg);
        if (need > smem) smem = need;
        const int per = a.step.per_wg * a.step.passes;
        const int wgs = (a.step.sel.rows * a.step.cpr + per - 1) / per;
        extra_rows = (wgs + a.n_split - 1) / a.n_split;
        aa.step.ref_rows = 0;
        if (a.step.ref_kt) {
            const int ref_wgs = a.B * a.H_kv * a.step.ref_blocks;
            aa.step.ref_rows = (ref_wgs + a.n_split - 1) / a.n_split;
            extra_rows += aa.step.ref_rows;
            if (KtildeShape<D>::kLdsBytes > smem) smem = KtildeShape<D>::kLdsBytes;
        }
    }
    const bool ref = step && a.step.ref_kt != nullptr;
    auto kern = ref ? attn_kernel<D, NT, true, false, true>
                    : step ? attn_kernel<D, NT, true> : a.nsa ? attn_kernel<D, NT, false, true> : attn_kernel<D, NT, false>;
    if (step) {
        hipLaunchKernelGGL(kern, dim3(a.n_split, tasks + extra_rows), dim3(a.waves * kWave), smem, s, aa);
        return hipGetLastError();
    }
    // grid rows are row groups; a launch covers at most 65535 of them
    for (int t0 = 0; t0 < tasks; t0 += kMaxGridRows) {
        aa.task0 = t0;
        hipLaunchKernelGGL(kern, dim3(a.n_split, min(kMaxGridRows, tasks - t0)), dim3(a.waves * kWave), smem, s, aa);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D, int NT>
static hipError_t grant_lds_t() {
    const void* kerns[4] = {reinterpret_cast<const void*>(attn_kernel<D, NT, false>),
                            reinterpret_cast<const void*>(attn_kernel<D, NT, true>),
                            reinterpret_cast<const void*>(attn_kernel<D, NT, false, true>),
                            reinterpret_cast<const void*>(attn_kernel<D, NT, true, false, true>)};
    for (const void* k : kerns) {
        const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsPerCU);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t attn_grant_lds() {
    hipError_t e = grant_lds_t<128, 1>();
    if (e == hipSuccess) e = grant_lds_t<128, 2>();
    if (e == hipSuccess) e = grant_lds_t<64, 1>();
    if (e == hipSuccess) e = grant_lds_t<64, 2>();
    return e;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    const hipError_t e = device_setup();
    if (e != hipSuccess) return e;
    const int rp = attn_rows_pad(a.C, a.G);
    if (a.d == 128) return rp == 16 ? launch_t<128, 1>(a, s) : launch_t<128, 2>(a, s);
    return rp == 16 ? launch_t<64, 1>(a, s) : launch_t<64, 2>(a, s);
}

}  // namespace sda
