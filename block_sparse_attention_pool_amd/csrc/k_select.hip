// Block scoring, exact top-k and block-set assembly.
//
// Scoring ([SparDA] note eq. (6) and (9), §4.2 step 2; [SSV] note, NSA
// selection-branch step 1): s_j = f . K~_j for every block of a row, fp32
// sums of exact bf16 x bf16 products.
// One workgroup per (batch, KV head, 256-block chunk, vector tile): the
// chunk of K~ (bf16, 256 bytes per block at d = 128) is streamed once and
// scored against every vector of the tile.  Sixteen lanes share a block row
// (one 16-byte load each at d = 128, 8 bytes at d = 64); the 16-lane partial
// sums are reduced with DPP.  The same
// kernel serves the G-head comparator, whose vectors are the G query heads
// of a KV group (eq. (8)).
//
// Selection as its own launch ([SparDA] eq. (3), eq. (6); §4.2 step 2), used
// when the in-launch selection below does not apply: one workgroup per row.
// Keys are the order-preserving uint32 image of the fp32 score; an 8-bit
// radix select over the candidates (blocks neither initial nor local) finds
// the k-th largest key, equal keys go to the lower block index, and an
// ordered compaction writes init U local U top-k ascending, padded with -1.
#include <math.h>

#include <type_traits>

#include "sda_device.hpp"
#include "sda_internal.h"
#include "sda_select_dev.hpp"

namespace sda {


int score_chunks(int NB_cap) { return (int)(((long long)NB_cap + kChunk - 1) / kChunk); }

// ---------------------------------------------------------------------------
// block-wide helpers (256 threads)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    const int lane = __lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_up(v, off, kWave);
        if (lane >= off) v += t;
    }
    return v;
}
// inclusive scan over the 256 threads in thread order; `sh` holds 4 words
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* sh) {
    const int lane = __lane_id(), w = threadIdx.x / kWave;
    v = wave_incl_scan(v);
    if (lane == kWave - 1) sh[w] = v;
    __syncthreads();
    uint32_t add = 0;
    for (int i = 0; i < w; ++i) add += sh[i];
    __syncthreads();
    return v + add;
}
__device__ __forceinline__ float block_reduce_max(float v, float* sh) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    if (__lane_id() == 0) sh[threadIdx.x / kWave] = v;
    __syncthreads();
    const float r = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
    __syncthreads();
    return r;
}
__device__ __forceinline__ float block_reduce_sum(float v, float* sh) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    if (__lane_id() == 0) sh[threadIdx.x / kWave] = v;
    __syncthreads();
    const float r = (sh[0] + sh[1]) + (sh[2] + sh[3]);
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------------------
// exact top-k + block set, one workgroup per row
// ---------------------------------------------------------------------------
// Exact top-k and block set of one row by one 256-lane workgroup.
template <int EPT>
__device__ __forceinline__ void select_row(const SelectArgs& a, int row) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t scan_sh[4];
    __shared__ uint32_t sh_digit, sh_gt;
    __shared__ uint32_t total;
    const int b = row / (a.NQ * a.H_kv);
    const int tid = threadIdx.x;
    const int nb = min((a.seq_len[b] + kBlock - 1) / kBlock, a.NB_cap);
    const int lo = min(a.n_init, nb);                   // candidates are [lo, hi)
    const int hi = max(lo, nb - a.n_local);
    const int ncand = hi - lo;
    const int k = min(a.top_k, ncand);
    const float* s = a.scores + (size_t)row * a.NB_cap;
    const int base = tid * EPT;                          // this thread owns [base, base+EPT)

    uint32_t key[EPT];
    uint64_t cand = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int j = base + i;
        const bool c = (j >= lo && j < hi);
        float sv = 0.f;
        if (c) sv = s[j];
        key[i] = c ? float_key(sv) : 0u;
        cand |= (uint64_t)c << i;
    }

    // radix select: find the k-th largest key among candidates
    uint32_t prefix = 0, pmask = 0;
    int krem = k;
    const bool partial = (k > 0 && k < ncand);
    if (partial) {
#pragma unroll 1
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            hist[tid] = 0;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < EPT; ++i)
                if (((cand >> i) & 1) && (key[i] & pmask) == prefix)
                    atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
            __syncthreads();
            // thread t looks at digit 255 - t: inclusive scan = count of digits >= it
            const uint32_t c = hist[255 - tid];
            const uint32_t incl = block_incl_scan(c, scan_sh);
            if (incl >= (uint32_t)krem && incl - c < (uint32_t)krem) {
                sh_digit = 255 - tid;
                sh_gt = incl - c;
            }
            __syncthreads();
            const uint32_t dg = sh_digit;
            krem -= (int)sh_gt;
            prefix |= dg << shift;
            pmask |= 255u << shift;
            __syncthreads();
        }
    }
    // prefix is now the k-th largest key; krem keys equal to it are taken,
    // lowest block index first
    uint32_t ties = 0;
    if (partial) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) ties += (((cand >> i) & 1) && key[i] == prefix) ? 1u : 0u;
    }
    const uint32_t ties_before = block_incl_scan(ties, scan_sh) - ties;

    const int n_init_eff = lo;                   // blocks [0, lo) are initial
    const int local_lo = max(0, nb - a.n_local);
    uint64_t take = 0;
    uint32_t tcount = ties_before;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int j = base + i;
        bool t = false;
        if (j < nb) {
            if (j < n_init_eff || j >= local_lo) t = true;
            else if ((cand >> i) & 1) {
                if (!partial) t = (k > 0);
                else if (key[i] > prefix) t = true;
                else if (key[i] == prefix) {
                    t = tcount < (uint32_t)krem;
                    ++tcount;
                }
            }
        }
        take |= (uint64_t)t << i;
    }
    const uint32_t mine = __popcll(take);
    const uint32_t incl = block_incl_scan(mine, scan_sh);
    uint32_t pos = incl - mine;
    int32_t* out = a.block_idx + (size_t)row * a.n_sel_max;
#pragma unroll
    for (int i = 0; i < EPT; ++i)
        if ((take >> i) & 1) {
            if (pos < (uint32_t)a.n_sel_max) out[pos] = base + i;
            ++pos;
        }
    if (tid == 255) total = incl;
    __syncthreads();
    const int tot = (int)min(total, (uint32_t)a.n_sel_max);
    for (int p = tot + tid; p < a.n_sel_max; p += 256) out[p] = -1;
    if (tid == 0) a.n_sel[row] = tot;
    __syncthreads();                        // the shared state may be reused by another row
}

template <int EPT>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
    select_row<EPT>(a, blockIdx.x);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
    const int ept = (a.NB_cap + 255) / 256;
    dim3 grid(a.rows), block(256);
    if (ept <= 1) hipLaunchKernelGGL(select_kernel<1>, grid, block, 0, s, a);
    else if (ept <= 2) hipLaunchKernelGGL(select_kernel<2>, grid, block, 0, s, a);
    else if (ept <= 4) hipLaunchKernelGGL(select_kernel<4>, grid, block, 0, s, a);
    else if (ept <= 8) hipLaunchKernelGGL(select_kernel<8>, grid, block, 0, s, a);
    else if (ept <= 16) hipLaunchKernelGGL(select_kernel<16>, grid, block, 0, s, a);
    else if (ept <= 32) hipLaunchKernelGGL(select_kernel<32>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(select_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
}

// vectors: [B, NQ, H_vec, D] bf16; K~ row (b, g) is scored by vectors
// (q, hv) with hv in [g*VPR, (g+1)*VPR).  out[((b*NQ + q)*H_vec + hv)*NB_cap + j]
// (out may be NULL when FUSED).
//
// FUSED (one vector per query, VPR = 1): the selection runs in the same launch
// in two levels.  Each chunk workgroup orders its 256 candidate blocks by the
// key (score, then lower block index): each wave sorts its 64 keys with a
// bitonic network across lanes and the sorted wave lists merge pairwise,
// leaving the chunk's best top_k keys, largest first, which go to `cand` with
// write-through stores.  Every chunk workgroup of a (kv row, vector tile)
// then bumps an agent-scope arrival counter; the last one merges the
// per-chunk sorted lists pairwise, round by round, and writes the block set.
// Each block lives in exactly one chunk and a global top-k block is within
// its chunk's top-k, so the merge is exact.
struct ScoreArgs {
    const uint16_t* vec;
    const uint16_t* kt;      // bf16 [B, H_kv, NB_cap, D]
    const int32_t* seq_len;
    float* out;
    int NQ, H_kv, VPR, NB_cap;
    float mult;
    SelectArgs sel;          // FUSED only
    uint64_t* cand;          // FUSED: [B*NQ*H_kv, chunks, top_k] keys
    int* counters;           // FUSED: [B*H_kv*vector tiles], zero between calls
};

constexpr int kScoresOnly = 0, kFusedSelect = 1;   // score_kernel modes

// Level 1 for one vector by one wave (workgroups of several vectors give each
// wave its own): lane l holds blocks l, l + 64, l + 128 and l + 192 of the
// chunk; each quarter is sorted across the lanes, then the quarters are
// merged pairwise (the lane-wise larger of one sorted list and the other
// reversed is bitonic and holds the pair's best 64), and the best K keys of
// the chunk are stored, largest first, as the four-wave level 1 does.
__device__ __forceinline__ uint64_t lane_reverse64(uint64_t x, int lane) {
    const int src = (lane ^ (kWave - 1)) << 2;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void wave_chunk_top_k(const float* sc, int j0, int lo, int hi, int K, uint64_t* dst,
                                                 int lane) {
    uint64_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = i * kWave + lane, j = j0 + t;
        q[i] = bitonic_sort<kWave, true>((j >= lo && j < hi) ? block_key(sc[t], j) : 0ull, lane);
    }
    const uint64_t r1 = lane_reverse64(q[1], lane), r3 = lane_reverse64(q[3], lane);
    const uint64_t a = bitonic_merge_desc<kWave>(q[0] > r1 ? q[0] : r1, lane);
    const uint64_t b = bitonic_merge_desc<kWave>(q[2] > r3 ? q[2] : r3, lane);
    const uint64_t rb = lane_reverse64(b, lane);
    const uint64_t c = bitonic_merge_desc<kWave>(a > rb ? a : rb, lane);
    if (lane < K) __hip_atomic_store(dst + lane, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Level 2 for one vector by one wave, when its nch chunk lists, each padded
// to P = 2^ceil(log2 K) keys, fit in the 64 lanes (lane = chunk * P + key):
// one sort of all of them across the lanes leaves the vector's best keys in
// the first lanes, the same keys the pairwise merges of the four-wave level
// 2 keep; then the block set is written as there (initial blocks, the chosen
// ids ascending, local blocks, -1 padding) and the vector's count.
__device__ __forceinline__ void wave_finish_row(const SelectArgs& s, const uint64_t* lists, int nch, int P,
                                                int vrow, int nb, int lane) {
    const int K = s.top_k;
    const int lo = min(s.n_init, nb);                      // candidates are [lo, hi)
    const int hi = max(lo, nb - s.n_local);
    const int kk = min(K, hi - lo);
    const int c = lane / P, p = lane - (lane / P) * P;
    uint64_t x = (c < nch && p < K) ? lists[c * K + p] : 0ull;
    x = bitonic_sort<kWave, true>(x, lane);
    int32_t* out = s.block_idx + (size_t)vrow * s.n_sel_max;
    if (kk > 0) {
        uint32_t id = lane < kk ? 0xFFFFFFFFu - (uint32_t)x : 0xFFFFFFFFu;
        id = bitonic_sort<kWave, false>(id, lane);
        if (lane < kk) out[lo + lane] = (int)id;
    }
    for (int i = lane; i < lo; i += kWave) out[i] = i;                          // initial blocks
    for (int i = lane; i < nb - hi; i += kWave) out[lo + kk + i] = hi + i;      // local blocks
    const int total = lo + kk + (nb - hi);
    for (int i = total + lane; i < s.n_sel_max; i += kWave) out[i] = -1;
    if (lane == 0) s.n_sel[vrow] = total;
}

// The selection inside a scoring launch: sc[v][t] holds the score of block
// j0 + t for vector v0 + v of kv row `row` = b * H_kv + g (the grid is
// (chunks, B * H_kv, vector tiles)).  Level 1 orders the chunk, level 2 (the
// last chunk workgroup of the row and tile to arrive) merges the chunk lists
// and writes the block sets; see the comment at ScoreArgs.
template <int NV>
__device__ __forceinline__ void select_tail(const SelectArgs& s, uint64_t* cand, int* counters,
                                            const float (*sc)[kChunk], int b, int g, int row, int NQ,
                                            int H_kv, int nvec, int v0, int j0, int nb) {
    __shared__ uint64_t wl[4 * kWave];                 // four sorted wave lists of 64
    __shared__ uint64_t bufA[kFusedTopK * kFusedChunks];
    __shared__ uint64_t bufB[kFusedTopK * kFusedChunks / 2];
    __shared__ int last;
    const int K = s.top_k;
    const int nch = gridDim.x;
    const int tid = threadIdx.x;
    const int lo = min(s.n_init, nb);                 // candidates are [lo, hi)
    const int hi = max(lo, nb - s.n_local);
    __syncthreads();                                   // sc complete

    // level 1: this chunk's best K keys, largest first (one vector: the four
    // waves together; several: a wave per vector, the vectors in parallel)
    if constexpr (NV == 1) {
        if (v0 < nvec) {                               // uniform over the workgroup
            uint64_t* dst = cand + ((size_t)((b * NQ + v0) * H_kv + g) * nch + blockIdx.x) * K;
            chunk_top_k(sc[0], j0, lo, hi, K, true, wl, dst, tid);
        }
    } else {
        const int lane = tid % kWave, wave = tid / kWave;
        for (int v = wave; v < NV; v += (int)blockDim.x / kWave) {
            const int vi = v0 + v;
            if (vi >= nvec) break;                     // uniform over the wave
            uint64_t* dst = cand + ((size_t)((b * NQ + vi) * H_kv + g) * nch + blockIdx.x) * K;
            wave_chunk_top_k(sc[v], j0, lo, hi, K, dst, lane);
        }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this workgroup's lists have landed
    __syncthreads();
    int* cnt = counters + (size_t)row * gridDim.z + blockIdx.z;
    if (tid == 0) {
        last = arrive(cnt) == nch - 1;
        if (last) acquire_agent();
    }
    __syncthreads();
    if (!last) return;

    // level 2: merge the nch chunk lists of each vector, then its block set
    if constexpr (NV == 1) {
        if (v0 < nvec) {
            // (the four-wave merges: one wave sorting all 8 x 32 keys of a
            // 128K row in four quarters made the launch slower, 15.9 against
            // 13.7 us)
            const int vrow = (b * NQ + v0) * H_kv + g;
            finish_row<true>(s, cand + (size_t)vrow * nch * K, nch, vrow, nb, bufA, bufB);
        }
    } else {
        // the lists of all the workgroup's vectors are requested in one batch
        // (when they fit) rather than one vector's after another's merge
        constexpr int kPreKeys = 2048;
        __shared__ uint64_t pre[kPreKeys];
        const int per = nch * K;
        const bool fits = NV * per <= kPreKeys;
        if (fits) {
            for (int i = tid; i < NV * per; i += blockDim.x) {
                const int v = i / per, vi = v0 + v;
                if (vi < nvec)
                    pre[i] = __hip_atomic_load(cand + (size_t)((b * NQ + vi) * H_kv + g) * per + (i - v * per),
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        }
        const int P = pow2_at_least(K);
        if (fits && nch * P <= kWave) {
            // a wave per vector, the vectors in parallel
            const int lane = tid % kWave, wave = tid / kWave;
            for (int v = wave; v < NV; v += (int)blockDim.x / kWave) {
                const int vi = v0 + v;
                if (vi >= nvec) break;                     // uniform over the wave
                wave_finish_row(s, pre + v * per, nch, P, (b * NQ + vi) * H_kv + g, nb, lane);
            }
        } else {
            for (int v = 0; v < NV; ++v) {
                const int vi = v0 + v;
                if (vi >= nvec) break;
                const int vrow = (b * NQ + vi) * H_kv + g;
                if (fits) finish_row<false>(s, pre + v * per, nch, vrow, nb, bufA, bufB);
                else finish_row<true>(s, cand + (size_t)vrow * per, nch, vrow, nb, bufA, bufB);
            }
        }
    }
    if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int NV, int MODE>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
    constexpr bool FUSED = MODE == kFusedSelect;
    constexpr bool LDS_SC = FUSED;
    constexpr int EPL = D / 16;             // bf16 elements per lane of one pooled key (16 lanes per key)
    using KLoad = typename std::conditional<EPL == 8, u32x4, u32x2>::type;
    const int row = blockIdx.y;             // b * H_kv + g
    const int b = row / a.H_kv, g = row - (row / a.H_kv) * a.H_kv;
    const int nb = min((a.seq_len[b] + kBlock - 1) / kBlock, a.NB_cap);
    const int j0 = blockIdx.x * kChunk;
    const int H_vec = a.H_kv * a.VPR;
    const int nvec = a.NQ * a.VPR;
    const int v0 = blockIdx.z * NV;
    const int lane = __lane_id();
    const int li = lane & 15;
    const int wave = threadIdx.x / kWave;
    __shared__ float sc[LDS_SC ? NV : 1][LDS_SC ? kChunk : 1];

    // this lane's slice of each vector (dims EPL*li .. EPL*li + EPL), loaded
    // raw beside the length read; converted once the key loads are out
    KLoad fw[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int vi = v0 + v;
        const int q = vi / a.VPR, hv = g * a.VPR + (vi - (vi / a.VPR) * a.VPR);
        fw[v] = vi < nvec ? *reinterpret_cast<const KLoad*>(a.vec + (((size_t)b * a.NQ + q) * H_vec + hv) * D +
                                                             li * EPL)
                          : KLoad{};
    }
    if (j0 < nb) {
        const uint16_t* ktr = a.kt + (size_t)row * a.NB_cap * D + li * EPL;
        constexpr int UNR = NV <= 2 ? 16 : 8;        // steps in flight
        constexpr int STEPS = kChunk / 16;           // 16 blocks per workgroup step
        float fv[NV][EPL];
        for (int s0 = 0; s0 < STEPS; s0 += UNR) {
            KLoad kv[UNR];
            int jj[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                jj[u] = j0 + (s0 + u) * 16 + wave * 4 + (lane >> 4);
                // past the length: re-read the last block (cached), result unused
                kv[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const KLoad*>(ktr + (size_t)min(jj[u], nb - 1) * D));
            }
            if (s0 == 0) {
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const uint32_t* wp = reinterpret_cast<const uint32_t*>(&fw[v]);
#pragma unroll
                    for (int i = 0; i < EPL / 2; ++i) {
                        fv[v][2 * i] = bf16lo(wp[i]);
                        fv[v][2 * i + 1] = bf16hi(wp[i]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const uint32_t* kp = reinterpret_cast<const uint32_t*>(&kv[u]);
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const float acc = key_dot<EPL>(fv[v], kp) * a.mult;
                    const int vi = v0 + v;
                    if (li == 0 && jj[u] < nb && vi < nvec) {
                        if constexpr (LDS_SC) sc[v][jj[u] - j0] = acc;
                        if (!FUSED || a.out) {
                            const int q = vi / a.VPR, hv = g * a.VPR + (vi - (vi / a.VPR) * a.VPR);
                            a.out[(((size_t)b * a.NQ + q) * H_vec + hv) * a.NB_cap + jj[u]] = acc;
                        }
                    }
                }
            }
        }
    }

    if constexpr (FUSED)
        select_tail<NV>(a.sel, a.cand, a.counters, sc, b, g, row, a.NQ, a.H_kv, nvec, v0, j0, nb);
}

// Pooled scoring ([SparDA] note: eq. (4) with kernel l and stride s, §4.4
// InfLLM-V2's inference compression l = 32, s = 16; §4.3 and fig. 3: the
// compressed scores are max-pooled onto the block grid).  Workgroup
// (chunk, kv row, query) scores every compressed entry whose window shares a
// token with one of its 256 blocks (256*64/s entries plus the (l-1)/s
// windows that reach in from the previous chunk: 1025 at l = 32, s = 16),
// 16 lanes per entry as in score_kernel, the scores kept in LDS; each lane
// then takes the max over its block's windows, and the selection runs as in
// score_kernel on those block scores.
constexpr int kPoolMaxEntries = kChunk * 64 / 8 + 8;      // stride >= 8, window <= 64
struct PoolArgs {
    int window, stride, NC_cap;
};

template <int D, int MODE>
__global__ __launch_bounds__(256) void pooled_score_kernel(ScoreArgs a, PoolArgs pa) {
    constexpr bool FUSED = MODE == kFusedSelect;
    constexpr int EPL = D / 16;
    constexpr int UNR = 16;                                 // entry steps in flight
    using KLoad = typename std::conditional<EPL == 8, u32x4, u32x2>::type;
    const int row = blockIdx.y;                             // b * H_kv + g
    const int b = row / a.H_kv, g = row - (row / a.H_kv) * a.H_kv;
    const int q = blockIdx.z;                               // one indexer vector per workgroup
    const int T = a.seq_len[b];
    const int nb = min((T + kBlock - 1) / kBlock, a.NB_cap);
    const int ne = min((T + pa.stride - 1) / pa.stride, pa.NC_cap);    // entries present
    const int j0 = blockIdx.x * kChunk;
    const int lane = __lane_id();
    const int li = lane & 15;
    const int wave = threadIdx.x / kWave;
    __shared__ float zc[kPoolMaxEntries];
    __shared__ float sc[1][kChunk];

    const KLoad fw = *reinterpret_cast<const KLoad*>(a.vec + (((size_t)b * a.NQ + q) * a.H_kv + g) * D + li * EPL);
    if (j0 < nb && ne > 0) {
        // entries overlapping blocks [j0, min(j0 + 256, nb)): j*s + l > 64*j0 and j*s < 64*min(...)
        const int lo_num = kBlock * j0 - pa.window + 1;
        const int e0 = lo_num > 0 ? (lo_num + pa.stride - 1) / pa.stride : 0;
        const int e1 = min(ne - 1, (kBlock * min(j0 + kChunk, nb) - 1) / pa.stride);
        const int cnt = e1 - e0 + 1;
        const uint16_t* ktr = a.kt + (size_t)row * pa.NC_cap * D + li * EPL;
        float fv[EPL];
        {
            const uint32_t* wp = reinterpret_cast<const uint32_t*>(&fw);
#pragma unroll
            for (int i = 0; i < EPL / 2; ++i) {
                fv[2 * i] = bf16lo(wp[i]);
                fv[2 * i + 1] = bf16hi(wp[i]);
            }
        }
        for (int s0 = 0; s0 * 16 < cnt; s0 += UNR) {
            KLoad kv[UNR];
            int jj[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                jj[u] = e0 + (s0 + u) * 16 + wave * 4 + (lane >> 4);
                // past the chunk's last entry: re-read that entry (cached), result unused
                kv[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const KLoad*>(ktr + (size_t)min(jj[u], e1) * D));
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const float acc = key_dot<EPL>(fv, reinterpret_cast<const uint32_t*>(&kv[u])) * a.mult;
                if (li == 0 && jj[u] <= e1) zc[jj[u] - e0] = acc;
            }
        }
        __syncthreads();
        // max-pool: block J = j0 + t takes the windows j*s < 64(J+1), j*s + l > 64J
        const int t = threadIdx.x;
        const int J = j0 + t;
        if (J < nb) {
            const int ln = kBlock * J - pa.window + 1;
            const int lo = max(e0, ln > 0 ? (ln + pa.stride - 1) / pa.stride : 0);
            const int hi = min(e1, (kBlock * J + kBlock - 1) / pa.stride);
            float m = -INFINITY;
            for (int e = lo; e <= hi; ++e) m = fmaxf(m, zc[e - e0]);
            sc[0][t] = m;
            if (a.out) a.out[(((size_t)b * a.NQ + q) * a.H_kv + g) * a.NB_cap + J] = m;
        }
    }
    if constexpr (FUSED)
        select_tail<1>(a.sel, a.cand, a.counters, sc, b, g, row, a.NQ, a.H_kv, a.NQ, q, j0, nb);
}

template <int D, int MODE>
static void launch_score_d(const ScoreArgs& a, int B, hipStream_t s) {
    const int nvec = a.NQ * a.VPR;
    const int nv = score_tile_vectors(nvec, a.NB_cap, B * a.H_kv);
    dim3 grid(score_chunks(a.NB_cap), B * a.H_kv, (nvec + nv - 1) / nv), block(256);
    switch (nv) {
        case 1: hipLaunchKernelGGL((score_kernel<D, 1, MODE>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((score_kernel<D, 2, MODE>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((score_kernel<D, 4, MODE>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((score_kernel<D, 8, MODE>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((score_kernel<D, 16, MODE>), grid, block, 0, s, a); break;
    }
}

// Vectors per scoring workgroup: up to 16 share one read of a chunk's
// compressed keys, but a workgroup selects for its vectors one after another,
// so tiles shrink (more workgroups, each key chunk read by several) while the
// grid would hold fewer than two workgroups per compute unit.
int score_tile_vectors(int nvec, int NB_cap, int rows) {
    int nv = 1;
    while (nv < nvec && nv < 16) nv *= 2;
    while (nv > 1 && (long long)score_chunks(NB_cap) * rows * (((long long)nvec + nv - 1) / nv) < 2LL * kCUs) nv /= 2;
    return nv;
}

int score_tiles(int NQ, int NB_cap, int rows) {
    const int nv = score_tile_vectors(NQ, NB_cap, rows);
    return (int)(((long long)NQ + nv - 1) / nv);
}

bool fused_select_ok(int NB_cap, int top_k) {
    return top_k >= 1 && top_k <= kFusedTopK && score_chunks(NB_cap) <= kFusedChunks;
}

hipError_t launch_score_select(const uint16_t* f, const uint16_t* kt, const SelectArgs& sel, int B, int d,
                               float* scores_opt, float* scores_ws, uint64_t* cand, int* counters,
                               hipStream_t s) {
    if (cand) {            // the selection inside the scoring launch
        ScoreArgs a{f, kt, sel.seq_len, scores_opt, sel.NQ, sel.H_kv, 1, sel.NB_cap, 1.f, sel, cand, counters};
        if (d == 128) launch_score_d<128, kFusedSelect>(a, B, s);
        else launch_score_d<64, kFusedSelect>(a, B, s);
        return hipGetLastError();
    }
    float* scores = scores_opt ? scores_opt : scores_ws;
    ScoreArgs a{f, kt, sel.seq_len, scores, sel.NQ, sel.H_kv, 1, sel.NB_cap, 1.f, sel, nullptr, nullptr};
    if (d == 128) launch_score_d<128, kScoresOnly>(a, B, s);
    else launch_score_d<64, kScoresOnly>(a, B, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SelectArgs sa = sel;
    sa.scores = scores;
    return launch_select(sa, s);
}

// pooled scores (one workgroup per chunk, kv row and query), then the
// selection: in the same launch with cand / counters, else a second launch
hipError_t launch_score_select_pooled(const uint16_t* f, const uint16_t* kt, const SelectArgs& sel, int B, int d,
                                      int window, int stride, int NC_cap, float* scores_opt, float* scores_ws,
                                      uint64_t* cand, int* counters, hipStream_t s) {
    const PoolArgs pa{window, stride, NC_cap};
    const dim3 grid(score_chunks(sel.NB_cap), B * sel.H_kv, sel.NQ), block(256);
    if (cand) {
        const ScoreArgs a{f, kt, sel.seq_len, scores_opt, sel.NQ, sel.H_kv, 1, sel.NB_cap, 1.f, sel, cand, counters};
        if (d == 128) hipLaunchKernelGGL((pooled_score_kernel<128, kFusedSelect>), grid, block, 0, s, a, pa);
        else hipLaunchKernelGGL((pooled_score_kernel<64, kFusedSelect>), grid, block, 0, s, a, pa);
        return hipGetLastError();
    }
    float* scores = scores_opt ? scores_opt : scores_ws;
    const ScoreArgs a{f, kt, sel.seq_len, scores, sel.NQ, sel.H_kv, 1, sel.NB_cap, 1.f, sel, nullptr, nullptr};
    if (d == 128) hipLaunchKernelGGL((pooled_score_kernel<128, kScoresOnly>), grid, block, 0, s, a, pa);
    else hipLaunchKernelGGL((pooled_score_kernel<64, kScoresOnly>), grid, block, 0, s, a, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SelectArgs sa = sel;
    sa.scores = scores;
    return launch_select(sa, s);
}

// ---------------------------------------------------------------------------
// G-head comparator: z = q_h . K~_j / tau, then s_j = sum_h softmax_j(z_h)
// ---------------------------------------------------------------------------
// Launch 1 (mh_score_kernel, one workgroup per 256-block chunk, KV row and
// query): the G heads of the KV group times the chunk's compressed keys as a
// small dense product on MFMA (keys x dims times dims x heads, four waves of
// 64 keys), z to the workspace plus, per head and chunk, the chunk max and the
// sum of exp(z - max).  Launch 2, one workgroup per (chunk, kv row, query):
// merges the row's chunk statistics into each head's softmax max M_h and
// normaliser L_h, forms s_j = sum_h exp(z_hj - M_h) / L_h for its 256 blocks
// and runs the in-launch selection on them (or writes the scores for the
// selection launch when that does not apply).
// floats of [z, padded to 64 floats][chunk statistics, padded to 64 floats]
size_t multihead_ws_floats(int B, int NQ, int H_q, int H_kv, int NB_cap) {
    (void)H_kv;
    const size_t z = ((size_t)B * NQ * H_q * NB_cap + 63) / 64 * 64;
    const size_t st = ((size_t)B * NQ * H_q * score_chunks(NB_cap) * 2 + 63) / 64 * 64;
    return z + st;
}

template <int D>
__global__ __launch_bounds__(256) void mh_score_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kt,
                                                       const int32_t* __restrict__ seq_len, float* __restrict__ z,
                                                       float* __restrict__ stats, int NQ, int H_q, int H_kv, int G,
                                                       int NB_cap, float mult, int stride) {
    constexpr int KS = D / 32;                          // MFMA k-steps over the head dim
    __shared__ float red[4][16];
    const int row = blockIdx.y;                         // b * H_kv + g
    const int b = row / H_kv, g = row - (row / H_kv) * H_kv;
    const int qi = blockIdx.z;
    const int nch = gridDim.x;
    const int j0 = blockIdx.x * kChunk;
    // compressed entries present (one per `stride` tokens; 64 for block keys)
    const int nb = min((seq_len[b] + stride - 1) / stride, NB_cap);
    const int lane = __lane_id(), li = lane & 15, lg = lane >> 4;
    const int wave = threadIdx.x / kWave;
    const size_t hrow0 = ((size_t)b * NQ + qi) * H_q + (size_t)g * G;   // first head row of the group
    const int jw = j0 + wave * kWave;                   // first key of this wave
    // S^T = K~ Q^T: A = 16 keys x 32 dims, B = 32 dims x 16 heads (heads past G
    // repeat the last one; their columns are never written)
    floatx4 sv[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sv[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (jw < nb) {
        u32x4 qf[KS], kf[4][KS];
        const uint16_t* qp = q + (hrow0 + min(li, G - 1)) * D + lg * 8;
        // whole 128-byte lines per load, then kswap to the A layout (lane l:
        // key jw + 16 mt + l % 16, dims 32 ks + 8 (l / 16))
        const char* kb = reinterpret_cast<const char*>(kt + (size_t)row * NB_cap * D) +
                         ((lane >> 4) + 4 * ((lane >> 3) & 1)) * 16;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int key = min(jw + mt * 16 + 8 * x + (lane & 7), nb - 1);   // past the length: a real key, result unused
#pragma unroll
                for (int h = 0; h < KS / 2; ++h) kf[mt][2 * h + x] = ldg16(kb + (size_t)key * D * 2 + h * 128);
            }
        kswap<KS>(kf);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = ldg16_cached(qp + ks * 32);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sv[mt] = mfma16x16x32(kf[mt][ks], qf[ks], sv[mt]);
    }
    // lane (li, lg) holds z of head li for keys jw + mt*16 + lg*4 + i
    float m = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sv[mt][i] *= mult;
            if (jw + mt * 16 + lg * 4 + i < nb) m = fmaxf(m, sv[mt][i]);
        }
    if (li < G) {
        float* zr = z + (hrow0 + li) * NB_cap;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int k0 = jw + mt * 16 + lg * 4;
            if (k0 + 3 < nb) {
                *reinterpret_cast<floatx4*>(zr + k0) = sv[mt];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (k0 + i < nb) zr[k0 + i] = sv[mt][i];
            }
        }
    }
    // chunk statistics per head: the max, then the sum of exp(z - max)
    m = cross4_max(m);
    if (lg == 0) red[wave][li] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0][li], red[1][li]), fmaxf(red[2][li], red[3][li]));
    float l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (jw + mt * 16 + lg * 4 + i < nb) l += expf(sv[mt][i] - M);
    }
    l = cross4_sum(l);
    __syncthreads();                                    // the maxima have been read
    if (lg == 0) red[wave][li] = l;
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        float* st = stats + ((hrow0 + h) * nch + blockIdx.x) * 2;
        st[0] = M;                                      // every wave of the workgroup computed the same M for h
        st[1] = (red[0][h] + red[1][h]) + (red[2][h] + red[3][h]);
    }
}

// Second comparator launch, one workgroup per (chunk, KV row, query): each
// head's softmax max and normaliser over the whole row, from the chunk
// statistics of the first launch; then s_j = sum over the heads of
// exp(z_hj - M_h) / L_h for this chunk's blocks, and the selection.  Every
// global load (this thread's z for all heads, the statistics, the length) is
// issued before the first wait, so the launch starts with one round trip.
constexpr int kMaxHeads = 16;
template <bool FUSED>
__global__ __launch_bounds__(256) void mh_select_kernel(const float* __restrict__ z, const float* __restrict__ stats,
                                                        SelectArgs sel, int H_q, int G, float* scores_out,
                                                        uint64_t* cand, int* counters) {
    __shared__ float sc[1][kChunk];
    __shared__ float pm[kMaxHeads][16], pl[kMaxHeads][16];   // per head: 16 partial (max, sum) pairs
    __shared__ float mh[kMaxHeads], il[kMaxHeads];
    const int row = blockIdx.y;                          // b * H_kv + g
    const int H_kv = sel.H_kv, NQ = sel.NQ, NB_cap = sel.NB_cap;
    const int b = row / H_kv, g = row - (row / H_kv) * H_kv;
    const int q = blockIdx.z;
    const int nch = gridDim.x;
    const int j0 = blockIdx.x * kChunk;
    const int tid = threadIdx.x;
    const size_t hrow0 = ((size_t)b * NQ + q) * H_q + (size_t)g * G;   // first head row of the group
    const int j = j0 + tid;
    // statistics: thread (sh, sc0) merges head sh's chunks sc0, sc0 + 16, ...;
    // the first pair is read as one 64-bit load before anything waits
    const int sh = tid >> 4, sc0 = tid & 15;
    const float* st = stats + (hrow0 + min(sh, G - 1)) * nch * 2;
    const bool has0 = sh < G && sc0 < nch;
    const uint64_t p0 = has0 ? *reinterpret_cast<const uint64_t*>(st + 2 * sc0) : 0;
    const int len = sel.seq_len[b];
    // z of this thread's block for every head (past the length or the
    // capacity: a real entry of the row, result unused)
    const float* zc = z + hrow0 * NB_cap + min(j, NB_cap - 1);
    float zv[kMaxHeads];
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h) zv[h] = (h < G) ? zc[(size_t)h * NB_cap] : 0.f;
    float m = -INFINITY, l = 0.f;
    auto merge_stat = [&](float cm, float cl) {
        if (cm != -INFINITY) {                           // an empty chunk adds nothing
            const float Mn = fmaxf(m, cm);
            l = l * expf(m - Mn) + cl * expf(cm - Mn);
            m = Mn;
        }
    };
    if (has0) merge_stat(__uint_as_float((uint32_t)p0), __uint_as_float((uint32_t)(p0 >> 32)));
    if (sh < G)
        for (int c = sc0 + 16; c < nch; c += 16) merge_stat(st[2 * c], st[2 * c + 1]);
    const int nb = min((len + kBlock - 1) / kBlock, NB_cap);
    pm[sh][sc0] = m;
    pl[sh][sc0] = l;
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) M = fmaxf(M, pm[tid][i]);
        float L = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (pm[tid][i] != -INFINITY) L += pl[tid][i] * expf(pm[tid][i] - M);
        mh[tid] = M;
        il[tid] = 1.f / L;
    }
    __syncthreads();
    float sv = 0.f;
    if (j < nb) {
#pragma unroll
        for (int h = 0; h < kMaxHeads; ++h)
            if (h < G) sv += expf(zv[h] - mh[h]) * il[h];
        const size_t srow = ((size_t)b * NQ + q) * H_kv + g;
        if (scores_out) scores_out[srow * NB_cap + j] = sv;
    }
    sc[0][tid] = sv;
    if constexpr (FUSED) select_tail<1>(sel, cand, counters, sc, b, g, row, NQ, H_kv, NQ, q, j0, nb);
}

hipError_t launch_multihead_select(const uint16_t* q, const uint16_t* kt, const SelectArgs& sel, int B, int H_q,
                                   int d, float tau, float* z, float* stats, float* scores_opt, float* scores_ws,
                                   uint64_t* cand, int* counters, hipStream_t s) {
    const int G = H_q / sel.H_kv;
    dim3 grid(score_chunks(sel.NB_cap), B * sel.H_kv, sel.NQ), block(256);
    if (d == 128)
        hipLaunchKernelGGL(mh_score_kernel<128>, grid, block, 0, s, q, kt, sel.seq_len, z, stats, sel.NQ, H_q,
                           sel.H_kv, G, sel.NB_cap, 1.f / tau, kBlock);
    else
        hipLaunchKernelGGL(mh_score_kernel<64>, grid, block, 0, s, q, kt, sel.seq_len, z, stats, sel.NQ, H_q,
                           sel.H_kv, G, sel.NB_cap, 1.f / tau, kBlock);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (cand && counters) {
        hipLaunchKernelGGL(mh_select_kernel<true>, grid, block, 0, s, z, stats, sel, H_q, G, scores_opt, cand,
                           counters);
        return hipGetLastError();
    }
    float* scores = scores_opt ? scores_opt : scores_ws;
    hipLaunchKernelGGL(mh_select_kernel<false>, grid, block, 0, s, z, stats, sel, H_q, G, scores, nullptr, nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    SelectArgs sa = sel;
    sa.scores = scores;
    return launch_select(sa, s);
}

// InfLLM-V2's selector on overlapping compressed keys ([SparDA] §4.3 eq. (8)
// and fig. 3: per-head softmax, sum over the G heads, max-pool onto the block
// grid; §4.4: kernel l = 32, stride s = 16 at inference).  Launch 1 is
// mh_score_kernel over the compressed entries (chunks of 256 entries);
// launch 2, one workgroup per (256-block chunk, KV row, query), merges each
// head's softmax statistics over all entry chunks, forms the entry sums
// s_e = sum_h exp(z_he - M_h) / L_h for every entry whose window overlaps
// its blocks (at most 256 * 64 / s + l / s of them, in LDS), takes for each
// block the max over its overlapping windows (the pooled index's reading of
// the overlap) and runs the selection as the other selectors do.
template <bool FUSED>
__global__ __launch_bounds__(256) void mh_pooled_select_kernel(const float* __restrict__ z,
                                                               const float* __restrict__ stats, SelectArgs sel,
                                                               int H_q, int G, int window, int stride, int NC_cap,
                                                               int n_ech, float* scores_out, uint64_t* cand,
                                                               int* counters) {
    __shared__ float sc[1][kChunk];
    __shared__ float se[kPoolMaxEntries];
    __shared__ float pm[kMaxHeads][16], pl[kMaxHeads][16];
    __shared__ float mh[kMaxHeads], il[kMaxHeads];
    const int row = blockIdx.y;
    const int H_kv = sel.H_kv, NQ = sel.NQ, NB_cap = sel.NB_cap;
    const int b = row / H_kv, g = row - (row / H_kv) * H_kv;
    const int q = blockIdx.z;
    const int j0 = blockIdx.x * kChunk;
    const int tid = threadIdx.x;
    const size_t hrow0 = ((size_t)b * NQ + q) * H_q + (size_t)g * G;
    const int sh = tid >> 4, sc0 = tid & 15;
    const float* st = stats + (hrow0 + min(sh, G - 1)) * n_ech * 2;
    float m = -INFINITY, l = 0.f;
    if (sh < G)
        for (int c = sc0; c < n_ech; c += 16) {
            const float cm = st[2 * c], cl = st[2 * c + 1];
            if (cm != -INFINITY) {
                const float Mn = fmaxf(m, cm);
                l = l * expf(m - Mn) + cl * expf(cm - Mn);
                m = Mn;
            }
        }
    pm[sh][sc0] = m;
    pl[sh][sc0] = l;
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) M = fmaxf(M, pm[tid][i]);
        float L = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (pm[tid][i] != -INFINITY) L += pl[tid][i] * expf(pm[tid][i] - M);
        mh[tid] = M;
        il[tid] = 1.f / L;
    }
    __syncthreads();
    const int len = sel.seq_len[b];
    const int nb = min((len + kBlock - 1) / kBlock, NB_cap);
    const int ne = min((len + stride - 1) / stride, NC_cap);
    float sv = 0.f;
    if (j0 < nb && ne > 0) {
        // entries overlapping blocks [j0, min(j0 + 256, nb)): j s + l > 64 j0 and j s < 64 min(...)
        const int lo_num = kBlock * j0 - window + 1;
        const int e0 = lo_num > 0 ? (lo_num + stride - 1) / stride : 0;
        const int e1 = min(ne - 1, (kBlock * min(j0 + kChunk, nb) - 1) / stride);
        for (int e = e0 + tid; e <= e1; e += blockDim.x) {
            const float* zc = z + hrow0 * NC_cap + e;
            float s = 0.f;
#pragma unroll
            for (int h = 0; h < kMaxHeads; ++h)
                if (h < G) s += expf(zc[(size_t)h * NC_cap] - mh[h]) * il[h];
            se[e - e0] = s;
        }
        __syncthreads();
        const int J = j0 + tid;
        if (J < nb) {
            const int ln = kBlock * J - window + 1;
            const int lo = max(e0, ln > 0 ? (ln + stride - 1) / stride : 0);
            const int hi = min(e1, (kBlock * J + kBlock - 1) / stride);
            float mx = -INFINITY;
            for (int e = lo; e <= hi; ++e) mx = fmaxf(mx, se[e - e0]);
            sv = mx;
            if (scores_out) scores_out[(((size_t)b * NQ + q) * H_kv + g) * NB_cap + J] = mx;
        }
    }
    sc[0][tid] = sv;
    if constexpr (FUSED) select_tail<1>(sel, cand, counters, sc, b, g, row, NQ, H_kv, NQ, q, j0, nb);
}

hipError_t launch_multihead_select_pooled(const uint16_t* q, const uint16_t* kt, const SelectArgs& sel, int B,
                                          int H_q, int d, float tau, int window, int stride, int NC_cap, float* z,
                                          float* stats, float* scores_opt, float* scores_ws, uint64_t* cand,
                                          int* counters, hipStream_t s) {
    const int G = H_q / sel.H_kv;
    const int n_ech = score_chunks(NC_cap);
    dim3 grid1(n_ech, B * sel.H_kv, sel.NQ), block(256);
    if (d == 128)
        hipLaunchKernelGGL(mh_score_kernel<128>, grid1, block, 0, s, q, kt, sel.seq_len, z, stats, sel.NQ, H_q,
                           sel.H_kv, G, NC_cap, 1.f / tau, stride);
    else
        hipLaunchKernelGGL(mh_score_kernel<64>, grid1, block, 0, s, q, kt, sel.seq_len, z, stats, sel.NQ, H_q,
                           sel.H_kv, G, NC_cap, 1.f / tau, stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid2(score_chunks(sel.NB_cap), B * sel.H_kv, sel.NQ);
    if (cand && counters) {
        hipLaunchKernelGGL(mh_pooled_select_kernel<true>, grid2, block, 0, s, z, stats, sel, H_q, G, window, stride,
                           NC_cap, n_ech, scores_opt, cand, counters);
        return hipGetLastError();
    }
    float* scores = scores_opt ? scores_opt : scores_ws;
    hipLaunchKernelGGL(mh_pooled_select_kernel<false>, grid2, block, 0, s, z, stats, sel, H_q, G, window, stride,
                       NC_cap, n_ech, scores, nullptr, nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    SelectArgs sa = sel;
    sa.scores = scores;
    return launch_select(sa, s);
}

}  // namespace sda
