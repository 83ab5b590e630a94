// Prefill selection: every query position of a prefill chunk chooses its own
// block set ([SparDA] eq. (3): the set is a function of the query position,
// with the local window next to it; the complexity section's eq. (16) counts
// one Forecast score per query token and compressed block).  Query r of the
// chunk sits at position p = pos0 + r and chooses as a decode step at length
// p + 1: blocks 0 .. p / 64 exist, the last n_local of them are local, the
// first n_init are initial, and top-k ranks the others by f_r . K~_j.  The
// caller keeps n_local >= 1, so every ranked block is complete at p.
//
// Workgroup = (tile of 64 queries, b * H_kv + g), four waves; wave w owns the
// tile's queries 16 w .. 16 w + 15.  Scores S^T[block][query] = K~[block] .
// F[query] on 16x16x32 bf16 MFMA: the compressed keys are the A operand (one
// 16-byte load per lane per 16 blocks x 32 dims), the wave's indexer vectors
// the B operand (loaded once).  Lane l then holds the scores of query l % 16
// for blocks 16 mt + 4 (l / 16) + i, i < 4: a query's scores sit in the four
// lanes l % 16 + 16 q, q < 4, at most kPrefillMaxBlocks of them (32 m-tiles
// of four registers).  The products of bf16 values are exact in fp32 and the
// sums are fp32, like the decode scorer's (only the order of summation
// differs).
//
// Top-k per query without sorting: the largest threshold tau on the
// order-preserving 32-bit score keys with at least k candidates at or above
// it, found one bit at a time from the top (up to 32 counting passes, each
// summed over the query's four lanes, until exactly k keys lie at or above
// the threshold so far); keys above tau are taken, and keys equal to
// tau fill the rest in ascending block order (ties to the lower block id).
// The block set (initial, local and chosen blocks) is written ascending by a
// prefix count over the blocks in id order.
#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

namespace {

constexpr int kPrefillTile = 64;                       // queries per workgroup
constexpr int kMT = kPrefillMaxBlocks / 16;            // score m-tiles per lane

// value of lane (lane - delta) of the same column (delta in {16, 32}); lanes
// below delta read their own value (callers mask them)
__device__ __forceinline__ int from_lane_below(int x, int delta) {
    const int lane = __lane_id();
    const int src = lane >= delta ? lane - delta : lane;
    return __builtin_amdgcn_ds_bpermute(src << 2, x);
}
__device__ __forceinline__ int from_lane(int x, int src) { return __builtin_amdgcn_ds_bpermute(src << 2, x); }

// sum over the four lanes of a query (l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ int sum4(int x) {
    const int lane = __lane_id();
    x += __builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, x);
    return x + __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, x);
}

// exclusive prefix over the query's four lanes in order q = lane / 16, and
// the four lanes' total
__device__ __forceinline__ int excl4(int x, int& total) {
    const int lane = __lane_id();
    const int lg = lane >> 4;
    int s = x;
    int t = from_lane_below(s, 16);
    s += lg >= 1 ? t : 0;
    t = from_lane_below(s, 32);
    s += lg >= 2 ? t : 0;                               // inclusive prefix
    total = from_lane(s, (lane & 15) + 48);
    return s - x;
}

template <int D>
__global__ __launch_bounds__(256) void prefill_select_kernel(PrefillSelectArgs a) {
    constexpr int KS = D / 32;
    const int row = blockIdx.y;                         // b * H_kv + g
    const int b = row / a.H_kv, g = row - (row / a.H_kv) * a.H_kv;
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int li = lane & 15, lg = lane >> 4;
    const int r0 = blockIdx.x * kPrefillTile + wave * 16;
    if (r0 >= a.NQ) return;                              // uniform over the wave
    const int r = min(r0 + li, a.NQ - 1);
    const bool own = r0 + li < a.NQ;                     // this lane's query exists
    const int T = a.seq_len[b];
    const int p = a.pos0 + r;                            // the query's position
    const bool live = own && p < T;                      // a query past the cache has no blocks
    const int nbq = live ? min(p / kBlock + 1, a.NB_cap) : 0;
    const int lo = min(a.n_init, nbq);                   // candidates are [lo, hi)
    const int hi = max(lo, nbq - a.n_local);
    const int k_eff = min(a.top_k, hi - lo);
    // blocks any query of the wave needs: scores below the largest hi, set
    // membership below the largest nbq (the wave's last query)
    const int p_last = a.pos0 + min(r0 + 15, a.NQ - 1);
    const int nb_w = max(0, min(min(p_last, T - 1) / kBlock + 1, a.NB_cap));
    const int hi_w = max(0, nb_w - a.n_local);
    const int nmt_s = (hi_w + 15) / 16;                  // m-tiles with scores
    const int nmt_o = (nb_w + 15) / 16;                  // m-tiles the block sets span

    // the wave's indexer vectors: B[k][n] = F[query n][dim k]
    u32x4 fb[KS];
    const uint16_t* fr = a.f + (((size_t)b * a.NQ + r) * a.H_kv + g) * D + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) fb[ks] = ldg16_cached(fr + ks * 32);

    // scores, as order-preserving keys; 0 (below every finite score's key)
    // for blocks that do not compete
    uint32_t key[kMT][4];
    const uint16_t* ktr = a.kt + (size_t)row * a.NB_cap * D + lg * 8;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        key[mt][0] = key[mt][1] = key[mt][2] = key[mt][3] = 0u;
        if (mt < nmt_s) {                                // uniform over the wave
            const uint16_t* kr = ktr + (size_t)min(mt * 16 + li, a.NB_cap - 1) * D;
            floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(ldg16(kr + ks * 32), fb[ks], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = mt * 16 + lg * 4 + i;
                key[mt][i] = (j >= lo && j < hi) ? float_key(acc[i]) : 0u;
            }
        }
    }

    // threshold: the largest tau with at least k_eff candidate keys >= tau.
    // Once exactly k_eff keys lie at or above the tau found so far, the lower
    // bits can only raise tau inside the gap below the k_eff-th key: the keys
    // at or above it, and so the chosen set, stay the same.  The wave stops
    // when all its queries are there (most of them well before bit 0).
    uint32_t tau = 0u;
    int at_tau = -1;                                     // keys >= tau, once tau has moved
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t t = tau | (1u << bit);
        int c = 0;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
            if (mt < nmt_s)
#pragma unroll
                for (int i = 0; i < 4; ++i) c += key[mt][i] >= t ? 1 : 0;
        c = sum4(c);
        if (c >= k_eff) {
            tau = t;
            at_tau = c;
        }
        if (__ballot(live && k_eff > 0 && at_tau != k_eff) == 0) break;
    }
    if (k_eff == 0) tau = 0xffffffffu;                   // nothing chosen (no finite key reaches it)
    int gt = 0, eq = 0;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
        if (mt < nmt_s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gt += key[mt][i] > tau ? 1 : 0;
                eq += key[mt][i] == tau ? 1 : 0;
            }
    gt = sum4(gt);
    eq = sum4(eq);
    const int need = k_eff - gt;                         // ties at tau to take, lowest block ids first
    const bool resolve = __ballot(live && eq > need) != 0;   // some query has more ties than room

    // the block set, ascending: position of block j = number of set blocks below j
    int32_t* out = a.block_idx + (((size_t)b * a.NQ + r) * a.H_kv + g) * a.n_sel_max;
    int base = 0, tie_base = 0;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        if (mt < nmt_o) {
            bool in[4];
            int tie_rank[4];
            if (resolve) {                               // rare: rank the ties of this m-tile
                int tcount = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) tcount += key[mt][i] == tau ? 1 : 0;
                int ttot;
                int texc = excl4(tcount, ttot);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    tie_rank[i] = tie_base + texc;
                    texc += key[mt][i] == tau ? 1 : 0;
                }
                tie_base += ttot;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) tie_rank[i] = 0;
            }
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = mt * 16 + lg * 4 + i;
                const bool chosen = key[mt][i] > tau || (key[mt][i] == tau && tie_rank[i] < need);
                in[i] = j < nbq && (j < lo || j >= hi || chosen);
                cnt += in[i] ? 1 : 0;
            }
            int tot;
            int pos = base + excl4(cnt, tot);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (in[i] && own) {
                    out[pos] = mt * 16 + lg * 4 + i;
                    ++pos;
                }
            base += tot;
        }
    }
    if (own) {
        for (int e = base + lg; e < a.n_sel_max; e += 4) out[e] = -1;
        if (lg == 0) a.n_sel[((size_t)b * a.NQ + r) * a.H_kv + g] = base;
    }
}

}  // namespace

hipError_t launch_prefill_select(const PrefillSelectArgs& a, int d, hipStream_t s) {
    dim3 grid((a.NQ + kPrefillTile - 1) / kPrefillTile, a.B * a.H_kv), block(256);
    if (d == 128) hipLaunchKernelGGL(prefill_select_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(prefill_select_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace sda
