// Row-tiled block-sparse attention: many query rows of one KV head share
// every block load.  Used for prefill, where every query position attends to
// its own block set ([SparDA] eq. (3) and (7) per position; the complexity
// section's eq. (15) counts k blocks of attention per query token), for
// exact verification of groups of two or more draft queries ([SSV] core
// mechanism 1: the union of the group's lists loaded once), and for NSA's
// three branches in exact mode ([SSV] NSA derivation steps 3-6: the
// compressed cache, the listed blocks and the window, gated).
//
// A workgroup owns a tile of Cq consecutive queries of one (b, g): R = Cq*G
// rows (query, head), 16 per wave, kept in registers for the whole walk (the
// Q fragments, the online-softmax state and the O accumulators).  The tile's
// block lists are merged into a bitmap in LDS (bit c of word j: query c lists
// block j).  The workgroup walks the set blocks in ascending order and loads
// each block's K and V once into LDS with direct loads, later blocks in
// flight while the current one is computed (two slots in prefill, up to four
// in verification; one barrier per block); every wave computes only the
// blocks that one of its queries lists and masks each row to its own list
// and, in prefill, to the tokens at or before its position.  A row belongs to
// one wave, so nothing is merged inside a workgroup: each wave normalises and
// writes its own rows.  Verification tiles may split their union among
// several workgroups (split-K), whose (m, l, o) partials the last to finish
// merges.  In the NSA mode each split walks one branch: a contiguous range
// of compressed blocks or of window blocks (every query of the tile sees
// them), or its share of the listed union; the merge keeps the branches
// apart and applies the gates.
//
// Per block and wave (16 rows):
//   S^T[tok][row] = K[tok][:] . Q[row][:]     16x16x32 bf16 MFMA; K is the A
//       operand, kept in LDS in operand order (the direct loads place each
//       lane's 16 bytes of every (m-tile, k-step) operand side by side), so
//       a wave reads an operand with one conflict-free 16-byte read at an
//       immediate offset.
//   online softmax per row in fp32 (exp2, scale * log2(e) folded in).
//   O^T[d][row] += V^T[d][tok] P^T[tok][row]  V^T from LDS transpose reads
//       of the decode's V tile layout; P split into two bf16 parts (hi + lo).
// The work is a dense contraction per block (R x 64 x d twice), so it runs on
// MFMA; what bounds it is how often a block is fetched, which the tile size
// sets (one fetch per tile instead of one per group of a few positions).
#include <limits.h>
#include <type_traits>
#include <math.h>

#include "sda_attn_dev.hpp"
#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

namespace {

// Blocks in flight per workgroup (slots of K and V in LDS).  Prefill keeps
// two (64 KB at d = 128), so that two workgroups share a compute unit: that
// measured faster (21 against 38 ms on the 32K prefill) than three or four
// slots with one workgroup.  Verification tiles walk a few blocks each
// between a prologue and a split merge; the host grants them as many slots
// as LDS holds beside the bitmap (up to four, one workgroup per compute
// unit), or two when there are enough tiles for two workgroups per compute
// unit.
constexpr int kPrefillBufs = 2;
constexpr int kMaxBufs = 4;
constexpr int kPre = 4;          // list entries per thread loaded in the prologue
constexpr float kLazyMax = 8.f;  // a row's reference maximum lags its true maximum by at most this (log2)

// the first block above j whose bitmap word is set (nb if none); wave-uniform
__device__ __forceinline__ int next_set(const uint32_t* bm, int j, int nb) {
    const int lane = __lane_id();
    for (int base = j + 1; base < nb; base += kWave) {
        const int idx = base + lane;
        const uint64_t bal = __ballot(idx < nb && bm[idx] != 0u);
        if (bal) return base + __builtin_ctzll(bal);
    }
    return nb;
}

// Bits k of the result: word w0 + k of the bitmap is set and below nb (16
// words from w0, a multiple of 16; the bitmap is allocated and cleared in
// whole multiples of 16 words).
__device__ __forceinline__ uint32_t set_words16(const uint32_t* bm, int w0, int nb) {
    if (w0 >= nb) return 0u;
    const u32x4* p = reinterpret_cast<const u32x4*>(bm + w0);
    const u32x4 x0 = p[0], x1 = p[1], x2 = p[2], x3 = p[3];
    uint32_t m = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        m |= (x0[k] != 0u ? 1u : 0u) << k;
        m |= (x1[k] != 0u ? 1u : 0u) << (4 + k);
        m |= (x2[k] != 0u ? 1u : 0u) << (8 + k);
        m |= (x3[k] != 0u ? 1u : 0u) << (12 + k);
    }
    const int valid = nb - w0;
    return valid >= 16 ? m : (m & ((1u << valid) - 1u));
}

// Wave sum of a per-lane count in [0, 16] and the sum over lower lanes, from
// one ballot per bit of the count.
__device__ __forceinline__ void wave_count_scan(int cnt, int& below, int& total) {
    below = 0;
    total = 0;
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {
        const uint64_t bal = __ballot((cnt >> bit) & 1);
        below += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))
                 << bit;
        total += __popcll(bal) << bit;
    }
}

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waves per workgroup: RW row waves (16 rows each), times two in verification
// tiles of up to 64 rows, whose two waves per 16 rows take the two 32-token
// halves of every block (each keeps its own softmax state; the pair merges
// at the end), so the chain of dependent work per block is halved.
template <int RW, bool GRP>
constexpr int tiled_ksplit() { return GRP && RW <= 4 ? 2 : 1; }

// NSA three-branch mode: the n_split workgroups of a tile go to the branches
// in proportion to their blocks, at least one to each branch that has any:
// first one split per non-empty branch, then each further split to the
// branch with the most blocks per split (the lower branch on a tie).  Every
// workgroup of the tile computes the same counts, so all agree without
// communicating.  With no block anywhere, all splits fall to the last branch.
__device__ __forceinline__ void nsa_assign(int S, int n0, int n1, int n2, int& s0, int& s1) {
    int c0 = n0 > 0, c1 = n1 > 0, c2 = n2 > 0;
    if (c0 + c1 + c2 == 0) {
        s0 = s1 = 0;
        return;
    }
    for (int k = c0 + c1 + c2; k < S; ++k) {
        // n_i / c_i against n_j / c_j by cross products (a branch with c = 0 has n = 0)
        const bool t01 = (long long)n0 * c1 >= (long long)n1 * c0;
        const int bx = t01 ? 0 : 1;
        const int nx = t01 ? n0 : n1, cx = t01 ? c0 : c1;
        const bool tx2 = (long long)nx * c2 >= (long long)n2 * cx;
        const int best = tx2 ? bx : 2;
        c0 += best == 0;
        c1 += best == 1;
        c2 += best == 2;
    }
    s0 = c0;
    s1 = c1;
}

// GRP: verification tiles (split-K, up to kMaxBufs slots); otherwise prefill
// (one workgroup per tile, kPrefillBufs slots).  NSA (with GRP): the
// three-branch mode.
template <int D, int RW, bool GRP, bool NSA = false>
__global__ __launch_bounds__((RW * tiled_ksplit<RW, GRP>() * 64)) void tiled_attn_kernel(TiledArgs a) {
    static_assert(GRP || !NSA, "the three-branch mode runs on verification tiles");
    constexpr int KSPLIT = tiled_ksplit<RW, GRP>();
    constexpr int W = RW * KSPLIT;               // waves
    constexpr int MTH = 4 / KSPLIT;              // QK m-tiles (16 tokens each) of a wave
    constexpr int KHH = 2 / KSPLIT;              // PV token halves (32 tokens each) of a wave
    constexpr int KS = D / 32;                   // QK k-steps
    constexpr int MTD = D / 16;                  // PV m-tiles over d
    constexpr int ROWB = D * 2;                  // bytes per token row
    constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
    constexpr int TILE = kBlock * ROWB;          // bytes of one K (or V) tile
    constexpr int NT = W * kWave;                // threads
    constexpr int PPL = TILE / 16 / NT;          // 16-byte pieces per lane per tile
    static_assert(4 * KS == W * PPL, "one K operand per direct load");
    static_assert(PPL >= 1, "at least one piece per lane");
    static_assert(4 * PPL < 64, "two blocks' loads fit the vmcnt counter");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    SDA_LDS char* lds = (SDA_LDS char*)smem;
    const int nbuf = GRP ? a.nbuf : kPrefillBufs;
    uint32_t* bm = reinterpret_cast<uint32_t*>(smem + (size_t)nbuf * 2 * TILE);

    // tile -> (b, g, query tile): consecutive workgroups go to the eight XCDs
    // in turn, so when the (b, g) pairs come in multiples of eight, XCD x
    // walks the query tiles of pairs x, x + 8, ... from the last one down (the
    // longest lists first), and tiles that share blocks share an L2
    const int S = GRP ? a.n_split : 1;
    const int split = GRP ? (int)(blockIdx.x % (unsigned)S) : 0;
    const int wg = GRP ? (int)(blockIdx.x / (unsigned)S) : (int)blockIdx.x;
    const int P = a.B * a.H_kv;
    int pair, tile;
    if ((P & 7) == 0) {
        const int slot = wg >> 3;
        pair = (slot / a.n_tiles) * 8 + (wg & 7);
        tile = a.n_tiles - 1 - slot % a.n_tiles;
    } else {
        pair = wg / a.n_tiles;
        tile = a.n_tiles - 1 - wg % a.n_tiles;
    }
    const int b = pair / a.H_kv, g = pair - (pair / a.H_kv) * a.H_kv;
    const int q0 = tile * a.Cq;
    const int Cg = min(a.Cq, a.NQ - q0);
    const int G = a.G;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int rw = wave % RW;                     // the wave's 16 rows
    const int th = wave / RW;                     // and its token share of each block
    const int li = lane & 15, lg = lane >> 4;
    // the length, the Q fragments and the tile's first list entries are all
    // requested before any of them is waited for
    const int T = min(ld_ro(a.seq_len + b), a.T_cap);

    // this lane's row and the wave's queries
    const int r = rw * 16 + li;
    const int c = r / G, h = r - (r / G) * G;
    const bool row_ok = c < Cg;
    const int cc = min(c, Cg - 1);
    const int cw0 = (rw * 16) / G, cw1 = min((rw * 16 + 15) / G, Cg - 1);
    const uint32_t wmask = cw1 >= cw0 ? (uint32_t)((((uint64_t)1 << (cw1 + 1)) - 1) & ~(((uint64_t)1 << cw0) - 1)) : 0u;
    const int lim = a.prefill ? a.pos0 + q0 + cc + 1 : INT_MAX;     // tokens below lim are visible
    const int lim_w = a.prefill ? a.pos0 + q0 + min(cw0, Cg - 1) + 1 : INT_MAX;   // the wave's smallest
    const bool wave_real = rw * 16 + 16 <= Cg * G;

    // Q fragments (B operand): row r, dims ks * 32 + lg * 8
    u32x4 qf[KS];
    {
        const uint16_t* qp = a.q + (((size_t)b * a.NQ + q0 + cc) * a.H_q + (size_t)g * G + h) * D + lg * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = ldg16(qp + ks * 32);
    }
    // entry i = (query i / n_sel_max, position i % n_sel_max) of the tile's
    // lists; the first kPre per thread are loaded here (indexes clamped into
    // the lists so the loads need no branch), the rest after the clear.  In
    // shared-representative mode (rep) a query takes the list of its group's
    // first query.
    const int nsm = a.n_sel_max;
    const int n_ent = Cg * nsm;
    const int nbmax = min(a.NB_cap, a.bm_words);         // blocks the bitmap holds
    int pj[kPre], pn[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int i = min((int)threadIdx.x + u * NT, n_ent - 1);
        const int qc = i / nsm, e = i - qc * nsm;
        const size_t row = ((size_t)b * a.NQ + q0 + (a.rep ? qc - qc % a.Cu : qc)) * a.H_kv + g;
        pn[u] = a.n_sel[row];
        pj[u] = a.block_idx[row * nsm + e];
    }

    // the tile's bitmap
    const int bm_alloc = (a.bm_words + 15) & ~15;
    for (int i = threadIdx.x; i < bm_alloc; i += NT) bm[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int i = (int)threadIdx.x + u * NT;
        const int qc = i / nsm, e = i - qc * nsm;
        const int n = min(max(pn[u], 0), nsm);
        if (i < n_ent && e < n && pj[u] >= 0 && pj[u] < nbmax) atomicOr(&bm[pj[u]], 1u << qc);
    }
    for (int i = threadIdx.x + kPre * NT; i < n_ent; i += NT) {
        const int qc = i / nsm, e = i - qc * nsm;
        const size_t row = ((size_t)b * a.NQ + q0 + (a.rep ? qc - qc % a.Cu : qc)) * a.H_kv + g;
        const int n = min(max(a.n_sel[row], 0), nsm);
        if (e < n) {
            const int j = a.block_idx[row * nsm + e];
            if (j >= 0 && j < nbmax) atomicOr(&bm[j], 1u << qc);
        }
    }
    int nb = (max(T, 0) + kBlock - 1) / kBlock;
    if (a.prefill) nb = min(nb, (a.pos0 + q0 + Cg - 1) / kBlock + 1);
    nb = min(nb, nbmax);
    // the Q fragments have landed: pass them through an asm so the compiler
    // counts no load of them against the direct loads below
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));
    __syncthreads();

    // the union's size and this split's share of it: entries [e0, e1) in
    // ascending block order; jn = the block of entry e0.  Lane l looks at
    // words 16 l .. 16 l + 15 of each 1024-word chunk.
    int n_u = 0, e0 = 0, e1 = 0, jn = nb;
    for (int base = 0; base < nb; base += 16 * kWave) {
        int below, tot;
        wave_count_scan(__popc(set_words16(bm, base + lane * 16, nb)), below, tot);
        n_u += tot;
    }
    // the split's branch (NSA), its block range and its share of the range:
    // tokens [lo, hi) of the rows kbase / vbase point at are visible, blocks
    // are walked below jend
    int branch = 1, bsplit = split, bS = S, n_s0 = 0, n_s1 = S;
    int lo = 0, hi = T, jend = nb;
    const size_t kvrow = (size_t)b * a.H_kv + g;
    const uint16_t* kbase = a.k + kvrow * a.T_cap * D;
    const uint16_t* vbase = a.v + kvrow * a.T_cap * D;
    if constexpr (NSA) {
        // compressed entries present at length T, and the window [T - window, T)
        const int ncmp = min((max(T, 0) + a.cmp_stride - 1) / a.cmp_stride, a.NC_cap);
        const int wlo = max(0, T - a.window);
        const int n_c = (ncmp + kBlock - 1) / kBlock;
        const int n_w = T > wlo ? (T - 1) / kBlock - wlo / kBlock + 1 : 0;
        nsa_assign(S, n_c, n_u, n_w, n_s0, n_s1);
        branch = split < n_s0 ? 0 : (split < n_s0 + n_s1 ? 1 : 2);
        bsplit = branch == 0 ? split : (branch == 1 ? split - n_s0 : split - n_s0 - n_s1);
        bS = branch == 0 ? n_s0 : (branch == 1 ? n_s1 : S - n_s0 - n_s1);
        if (branch != 1) {
            const int cnt = branch == 0 ? n_c : n_w;
            const int rb = branch == 0 ? 0 : wlo / kBlock;
            if (branch == 0) {
                kbase = a.kc + kvrow * a.NC_cap * D;
                vbase = a.vc + kvrow * a.NC_cap * D;
                hi = ncmp;
            } else {
                lo = wlo;
            }
            e0 = bS > 0 ? (int)(((long long)bsplit * cnt) / bS) : 0;
            e1 = bS > 0 ? (int)(((long long)(bsplit + 1) * cnt) / bS) : 0;
            jn = rb + e0;                                // = jend when the share is empty
            jend = rb + e1;
        }
    }
    if (branch == 1) {
        e0 = (int)(((long long)bsplit * n_u) / bS);
        e1 = (int)(((long long)(bsplit + 1) * n_u) / bS);
    }
    if (branch == 1 && e0 < e1) {
        int seen = 0;
        for (int base = 0; base < nb; base += 16 * kWave) {
            const int w0 = base + lane * 16;
            uint32_t m16 = set_words16(bm, w0, nb);
            const int cnt = __popc(m16);
            int below, tot;
            wave_count_scan(cnt, below, tot);
            if (e0 < seen + tot) {                               // wave-uniform
                const int k = e0 - seen - below;                 // rank inside this lane's words
                const bool own = k >= 0 && k < cnt;
                if (own)
                    for (int t = k; t > 0; --t) m16 &= m16 - 1u;     // drop the lower set bits
                const int pos = own ? w0 + __builtin_ctz(m16) : 0;
                const uint64_t ob = __ballot(own);
                jn = __builtin_amdgcn_readlane(pos, __builtin_ctzll(ob));
                break;
            }
            seen += tot;
        }
    }
    // union_count: a tile of one group writes its union's size here; a tile
    // of several groups of Cu queries counts each group's union from the
    // bitmap after its walk (group_unions below)
    if (GRP && a.union_count && split == 0 && a.Cu == a.Cq && threadIdx.x == 0)
        a.union_count[((size_t)b * a.n_ugroups + tile) * a.H_kv + g] = n_u;
    // wave w counts the union of groups w, w + W, ... of the tile's Cu-query
    // groups (the bitmap is intact until the split merge's flag)
    auto group_unions = [&]() {
        if (!GRP || !a.union_count || split != 0 || a.Cu >= a.Cq || a.Cu < 2) return;   // groups of one: no count
        for (int u = wave; u * a.Cu < Cg; u += W) {
            const int c0 = u * a.Cu, c1 = min(c0 + a.Cu, Cg);
            const uint32_t gm = (uint32_t)((((uint64_t)1 << c1) - 1) & ~(((uint64_t)1 << c0) - 1));
            int cnt = 0;
            for (int base = 0; base < nb; base += kWave) {
                const int i = base + lane;
                cnt += __popcll(__ballot(i < nb && (bm[i] & gm) != 0u));
            }
            if (lane == 0)
                a.union_count[((size_t)b * a.n_ugroups + (size_t)tile * (a.Cq / a.Cu) + u) * a.H_kv + g] = cnt;
        }
    };
    // the block after j in the walk: the bitmap's next set word, or j + 1 in
    // a block range
    auto next_blk = [&](int j) { return (NSA && branch != 1) ? j + 1 : next_set(bm, j, nb); };
    auto issue = [&](int j, int slot) {
        const int tmax = min(kBlock - 1, hi - 1 - j * kBlock);
        const char* kb = reinterpret_cast<const char*>(kbase + (size_t)j * kBlock * D);
        const char* vb = reinterpret_cast<const char*>(vbase + (size_t)j * kBlock * D);
        SDA_LDS char* kl = lds + (size_t)slot * 2 * TILE;
        SDA_LDS char* vl = kl + TILE;
        // K: load i of this wave fills operand op = wave + W i, i.e. m-tile
        // op / KS and k-step op % KS; lane l brings token tok_of(mt, l % 16),
        // dims 32 ks + 8 (l / 16) .. + 7
#pragma unroll
        for (int i = 0; i < PPL; ++i) {
            const int op = wave + W * i;
            const int mt = op / KS, ks = op - (op / KS) * KS;
            const int tr = min(tok_of(mt, li), tmax);
            lds_dma16_async(kb + (size_t)tr * ROWB + ks * 64 + lg * 16, kl + op * kWave * 16);
        }
#pragma unroll
        for (int i = 0; i < PPL; ++i) {
            const int base = (wave + W * i) * kWave;
            const int pi = base + lane;
            const int t = pi / CPR, pc = pi - (pi / CPR) * CPR;
            const int tr = min(t, tmax);
            lds_dma16_async(vb + (size_t)tr * ROWB + ((pc << 4) ^ (VTile<D>::perm(t) << 5)), vl + base * 16);
        }
    };

    floatx4 o[MTD];
#pragma unroll
    for (int i = 0; i < MTD; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float csc = a.scale_log2;
    const int v_lane = (lg * 8 + (li >> 2)) * ROWB + (li & 3) * 8;   // row 8 lg + li / 4, column bytes
    const int v_perm = VTile<D>::perm(lg * 8 + (li >> 2));

    // the work of block j, whose K and V sit in `slot`
    auto compute = [&](int j, int slot) {
        const uint32_t mk = (NSA && branch != 1) ? ~0u : bm[j];   // every query sees a range block
        if (mk & wmask) {                                    // wave-uniform
            SDA_LDS const char* kl = lds + (size_t)slot * 2 * TILE;
            SDA_LDS const char* vl = kl + TILE;
            const int nvalid = min(kBlock, hi - j * kBlock);
            // every row of the wave is a real row that lists j and sees all of it
            const bool full = nvalid == kBlock && wave_real && (mk & wmask) == wmask && j * kBlock + kBlock <= lim_w &&
                              (!NSA || j * kBlock >= lo);
            // m-tiles th * MTH .. (tokens 32 th .. 32 th + 31 when split)
            floatx4 s[MTH];
            SDA_LDS const char* kq = kl + lane * 16 + th * (MTH * KS * kWave * 16);
#pragma unroll
            for (int mt = 0; mt < MTH; ++mt) {
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const u32x4 ka = *reinterpret_cast<SDA_LDS const u32x4*>(kq + (mt * KS + ks) * kWave * 16);
                    acc = mfma16x16x32(ka, qf[ks], acc);
                }
                s[mt] = acc;
            }
            if (!full) {
                // output i of m-tile mg is token tok_of(mg, 4 lg + i) = 8 lg + e(mg, i):
                // it counts when e < thr
                const bool live = row_ok && ((mk >> cc) & 1u);
                const int thr = (live ? min(nvalid, lim - j * kBlock) : 0) - lg * 8 - th * 32;
#pragma unroll
                for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!((mt >> 1) * 32 + (mt & 1) * 4 + i < thr)) s[mt][i] = -INFINITY;
                if constexpr (NSA) {
                    // the window's first block: tokens below lo are not in it
                    const int lthr = lo - j * kBlock - lg * 8 - th * 32;
#pragma unroll
                    for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if ((mt >> 1) * 32 + (mt & 1) * 4 + i < lthr) s[mt][i] = -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < MTH; ++mt) mx = fmaxf(mx, fmaxf(fmaxf(s[mt][0], s[mt][1]), fmaxf(s[mt][2], s[mt][3])));
            mx = cross4_max(mx) * csc;
            // the reference maximum of a row moves only when a block's
            // maximum exceeds it by more than kLazyMax (log2 units): most
            // blocks then skip the rescale of o, and the probabilities stay
            // below 2^kLazyMax (fp32 sums; P keeps its hi + lo bf16 parts)
            const bool grow = m_run == -INFINITY || mx > m_run + kLazyMax;
            const float m_new = grow ? fmaxf(m_run, mx) : m_run;
            const float m_use = m_new != -INFINITY ? m_new : 0.f;
            float psum = 0.f;
#pragma unroll
            for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[mt][i], csc, -m_use));
                    s[mt][i] = p;
                    psum += p;
                }
            psum = cross4_sum(psum);
            const bool rescale = grow && m_run != -INFINITY;
            if (__ballot(rescale)) {                             // wave-uniform
                const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < MTD; ++i) {
                    o[i][0] *= alpha;
                    o[i][1] *= alpha;
                    o[i][2] *= alpha;
                    o[i][3] *= alpha;
                }
            }
            l_run += psum;
            m_run = m_new;
            u32x4 pf[KHH], pl[KHH];
#pragma unroll
            for (int kh = 0; kh < KHH; ++kh)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float p0 = s[2 * kh + (w >> 1)][(w & 1) * 2];
                    const float p1 = s[2 * kh + (w >> 1)][(w & 1) * 2 + 1];
                    const bf16x2 hi = {(__bf16)p0, (__bf16)p1};
                    const bf16x2 lo = {(__bf16)(p0 - (float)hi[0]), (__bf16)(p1 - (float)hi[1])};
                    pf[kh][w] = __builtin_bit_cast(uint32_t, hi);
                    pl[kh][w] = __builtin_bit_cast(uint32_t, lo);
                }
            // V^T operands: token t = 32 kh + 8 lg + 4 hh + li / 4, whose chunk
            // permutation perm(t) is the lane's own (kh and hh do not enter it),
            // so one address per md and the (kh, hh) offsets are immediates
#pragma unroll
            for (int md = 0; md < MTD; ++md) {
                SDA_LDS const char* vq = vl + v_lane + ((md ^ v_perm) << 5) + th * (32 * ROWB);
#pragma unroll
                for (int kh = 0; kh < KHH; ++kh) {
                    u32x4 va;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const v4i16 rr = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (SDA_LDS v4i16*)(vq + (kh * 32 + hh * 4) * ROWB));
                        const uint2 u = __builtin_bit_cast(uint2, rr);
                        va[2 * hh] = u.x;
                        va[2 * hh + 1] = u.y;
                    }
                    o[md] = mfma16x16x32(va, pf[kh], o[md]);
                    o[md] = mfma16x16x32(va, pl[kh], o[md]);
                }
            }
        }
    };

    // nbuf slots, one barrier per block: blocks go to slots in turn and up to
    // nbuf - 1 are in flight.  At the top of iteration it the wave waits for
    // its share of block it (the loads of the blocks issued after it may stay
    // in flight: they are the last ones it issued), and the barrier then says
    // both that all of it has landed and that every wave is done with the
    // block before it, whose slot the next block's loads fill while it is
    // computed.
    int to_issue = e1 - e0;                 // blocks of this split not yet issued
    if constexpr (!GRP) {
        // two slots: the block issued in one iteration is computed in the next
        auto advance = [&](int j) { return --to_issue > 0 ? next_blk(j) : nb; };
        int j = jn;
        if (j < nb) {
            issue(j, 0);
            jn = advance(j);
        }
        for (int it = 0; j < nb; ++it) {
            const int slot = it & 1;
            vm_wait<0>();
            barrier_lds();
            const int jnext = jn;
            if (jnext < nb) {
                issue(jnext, slot ^ 1);
                jn = advance(jnext);
            }
            compute(j, slot);
            j = jnext;
        }
    } else {
        int j_iss = jn, n_iss = 0, islot = 0;   // the next block to issue, blocks issued, its slot
        int ring0 = jend, ring1 = jend, ring2 = jend, ring3 = jend;   // the block in each slot (wave-uniform)
        auto issue_next = [&]() {
            issue(j_iss, islot);
            ring0 = islot == 0 ? j_iss : ring0;
            ring1 = islot == 1 ? j_iss : ring1;
            ring2 = islot == 2 ? j_iss : ring2;
            ring3 = islot == 3 ? j_iss : ring3;
            ++n_iss;
            islot = islot + 1 == nbuf ? 0 : islot + 1;
            j_iss = --to_issue > 0 ? next_blk(j_iss) : jend;
        };
        for (int s0 = 0; s0 < nbuf - 1 && j_iss < jend; ++s0) issue_next();
        const int share = e1 - e0;
        int slot = 0;
        for (int it = 0; it < share; ++it) {
            const int ahead = n_iss - it - 1;                // blocks issued after this one, at most nbuf - 2
            if (ahead >= 2) vm_wait<4 * PPL>();
            else if (ahead == 1) vm_wait<2 * PPL>();
            else vm_wait<0>();
            barrier_lds();
            const int j = slot == 0 ? ring0 : slot == 1 ? ring1 : slot == 2 ? ring2 : ring3;
            if (j_iss < jend) issue_next();
            compute(j, slot);
            slot = slot + 1 == nbuf ? 0 : slot + 1;
        }
    }

    if constexpr (KSPLIT == 2) {
        // the two waves of each 16 rows merge their token halves: the second
        // puts (m, l, o) in LDS (the slots are free once every wave is past
        // the barrier), the first reads them with the same lane layout
        float* xo = reinterpret_cast<float*>(smem);                     // [RW][MTD][64] x 4
        float* xm = xo + RW * MTD * kWave * 4;                          // [RW][64]
        float* xl = xm + RW * kWave;
        __syncthreads();
        if (th == 1) {
#pragma unroll
            for (int md = 0; md < MTD; ++md)
                *reinterpret_cast<floatx4*>(xo + ((rw * MTD + md) * kWave + lane) * 4) = o[md];
            xm[rw * kWave + lane] = m_run;
            xl[rw * kWave + lane] = l_run;
        }
        __syncthreads();
        if (th == 0) {
            const float m2 = xm[rw * kWave + lane], l2 = xl[rw * kWave + lane];
            const float M = fmaxf(m_run, m2);
            const float a1 = M != -INFINITY ? __builtin_amdgcn_exp2f(m_run - M) : 0.f;
            const float a2 = M != -INFINITY ? __builtin_amdgcn_exp2f(m2 - M) : 0.f;
            l_run = l_run * a1 + l2 * a2;
            m_run = M;
#pragma unroll
            for (int md = 0; md < MTD; ++md) {
                const floatx4 o2 = *reinterpret_cast<const floatx4*>(xo + ((rw * MTD + md) * kWave + lane) * 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[md][i] = o[md][i] * a1 + o2[i] * a2;
            }
        }
    }

    if (!GRP || (!NSA && S == 1)) {
        group_unions();
        if (th == 0 && row_ok && r < Cg * G) {
            const size_t oi = ((size_t)b * a.NQ + q0 + c) * a.H_q + (size_t)g * G + h;
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
            for (int md = 0; md < MTD; ++md)
                *reinterpret_cast<floatx4*>(&a.out[oi * D + md * 16 + lg * 4]) =
                    floatx4{o[md][0] * inv, o[md][1] * inv, o[md][2] * inv, o[md][3] * inv};
            if (lg == 0 && a.lse) a.lse[oi] = l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
        }
        return;
    }

    if constexpr (GRP) {
    // ---- split-K: publish (m, l, o) of every row, the last workgroup merges ----
    // Agent-scope stores (write-through: the merging workgroup may sit on
    // another XCD), completed before one agent-scope increment per workgroup;
    // the last arrival acquires and reads them with agent-scope loads.
    constexpr int RP = RW * 16;                                  // rows of a tile
    constexpr int RPW = RP / W;                                  // rows each wave merges
    const size_t tg = (size_t)pair * a.n_tiles + tile;          // this tile
    if (th == 0) {
        const size_t pr = (tg * S + split) * RP + r;
        // o: 16 bytes per lane and m-tile (4 lanes fill 64 contiguous bytes of a row)
        float* pbase = a.part_o + (tg * S + split) * RP * D;
#pragma unroll
        for (int md = 0; md < MTD; ++md) st_agent16(pbase, (uint32_t)((r * D + md * 16 + lg * 4) * 4), o[md]);
        if (lg == 0)
            __hip_atomic_store(reinterpret_cast<uint64_t*>(a.part_ml + pr * 2),
                               ((uint64_t)__float_as_uint(l_run) << 32) | __float_as_uint(m_run), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    group_unions();                         // while the stores above are on their way
    // the flag lives in the bitmap's first word: every wave is past its last
    // read of the bitmap at the barrier below (the kernel uses no static LDS,
    // so that the whole 160 KB can be granted to the dynamic part)
    volatile int* s_last = reinterpret_cast<volatile int*>(bm);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const int last = arrive(a.counters + tg) == S - 1;
        if (last) acquire_agent();
        *s_last = last;
    }
    __syncthreads();
    if (!*s_last) return;
    // each wave merges RPW rows.  Lane r (and r + RPW, ...) reads row r's
    // (m, l) of every split and forms the row's maximum, scale factors and
    // normaliser; the o partials are read one row per load (lane = D / 64
    // adjacent columns, so a load covers the row's contiguous bytes), every
    // load of a batch of splits in flight together (indexes clamped to the
    // last split, so no branch separates them), and summed in split order
    // with the row's factor taken from lane r.
    constexpr int CPL = D / kWave;                               // columns per lane
    using ovec = typename std::conditional<CPL == 2, uint64_t, uint32_t>::type;
    constexpr int kMergeBatch = RPW <= 8 ? 8 : 4;
    const int r16 = lane % RPW;
    const size_t row0 = tg * S * RP + (size_t)wave * RPW;       // split 0, the wave's first row
    const uint64_t* pml = reinterpret_cast<const uint64_t*>(a.part_ml) + row0 + r16;
    const ovec* pob = reinterpret_cast<const ovec*>(a.part_o + row0 * D) + lane;   // rows kWave ovecs apart
    // one batch of kMergeBatch splits: their (m, l) words and o rows all in
    // flight together, then the batch folded into the running (M, L, acc) by
    // log-sum-exp (a single batch, the usual case, is the plain merge)
    // lane r16's row of the output: whether it is a real row, and its place in out / lse
    auto row16 = [&](bool& ok, size_t& oi) {
        const int mr = wave * RPW + r16;
        const int mcq = mr / G, mh = mr - (mr / G) * G;
        ok = mcq < Cg && mr < Cg * G;
        oi = ((size_t)b * a.NQ + q0 + min(mcq, Cg - 1)) * a.H_q + (size_t)g * G + mh;
    };
    float M = -INFINITY, L = 0.f, acc[RPW][CPL];
    if constexpr (NSA) {
        // the gated sum: each branch's splits (bnd[bi] .. bnd[bi + 1]) merged and
        // normalised, then o = g_c o_c + g_s o_s + g_w o_w, one lse per branch
        // (natural log, -inf for a branch that saw no token)
        const int bnd[4] = {0, n_s0, n_s0 + n_s1, S};
        float gt[3], oacc[RPW][CPL];
        bool ok16;
        size_t oi16;
        row16(ok16, oi16);
#pragma unroll
        for (int bi = 0; bi < 3; ++bi) gt[bi] = ok16 ? a.gates[oi16 * 3 + bi] : 0.f;
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
            for (int cc2 = 0; cc2 < CPL; ++cc2) oacc[rr][cc2] = 0.f;
        // a batch of splits: their (m, l) words and o rows, batch entry i = split base + i
        uint64_t w[kMergeBatch];
        ovec ov[kMergeBatch][RPW];
        auto load_batch = [&](int base, int s_hi) {
#pragma unroll
            for (int i = 0; i < kMergeBatch; ++i) {
                const size_t sp = (size_t)min(base + i, s_hi - 1) * RP;
                w[i] = __hip_atomic_load(pml + sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                for (int rr = 0; rr < RPW; ++rr)
                    ov[i][rr] = __hip_atomic_load(pob + (sp + rr) * kWave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        };
        // with at most one batch of splits, every split of every branch is
        // loaded at once and each branch folds its own entries of that batch
        const bool one_batch = S <= kMergeBatch;
        if (one_batch) load_batch(0, S);
#pragma unroll
        for (int bi = 0; bi < 3; ++bi) {
            if (bi > 0) {
                M = -INFINITY;
                L = 0.f;
            }
#pragma unroll
            for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
                for (int cc2 = 0; cc2 < CPL; ++cc2) acc[rr][cc2] = 0.f;
            const int s_lo = bnd[bi], s_hi = bnd[bi + 1];
            for (int s0 = s_lo; s0 < s_hi; s0 += kMergeBatch) {
                if (!one_batch) load_batch(s0, s_hi);
                const int base = one_batch ? 0 : s0;
                // entry i belongs to this pass when split base + i lies in [s0, s_hi)
                float Mb = M;
#pragma unroll
                for (int i = 0; i < kMergeBatch; ++i)
                    if (!one_batch || (i >= s0 && i < s_hi)) Mb = fmaxf(Mb, __uint_as_float((uint32_t)w[i]));
                if (s0 > s_lo) {
                    // earlier batches: rescale every row by its own factor (lane r's
                    // row r; 1 while the row has seen nothing), in every lane
                    const float al = (M != -INFINITY && Mb != M) ? __builtin_amdgcn_exp2f(M - Mb) : 1.f;
                    L *= al;
#pragma unroll
                    for (int rr = 0; rr < RPW; ++rr) {
                        const float alr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), rr));
#pragma unroll
                        for (int cc2 = 0; cc2 < CPL; ++cc2) acc[rr][cc2] *= alr;
                    }
                }
                M = Mb;
#pragma unroll
                for (int i = 0; i < kMergeBatch; ++i) {
                    if (base + i >= s0 && base + i < s_hi) {
                        const float ms = __uint_as_float((uint32_t)w[i]);
                        const float ls = __uint_as_float((uint32_t)(w[i] >> 32));
                        // 0 for an empty split, and for every split of a row no split saw
                        const float sc = M != -INFINITY ? __builtin_amdgcn_exp2f(ms - M) : 0.f;
                        L += ls * sc;
#pragma unroll
                        for (int rr = 0; rr < RPW; ++rr) {
                            const float scr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), rr));
                            if constexpr (CPL == 2) {
                                acc[rr][0] += __uint_as_float((uint32_t)ov[i][rr]) * scr;
                                acc[rr][1] += __uint_as_float((uint32_t)((uint64_t)ov[i][rr] >> 32)) * scr;
                            } else {
                                acc[rr][0] += __uint_as_float((uint32_t)ov[i][rr]) * scr;
                            }
                        }
                    }
                }
            }
            {
                const float wgt = L > 0.f ? gt[bi] / L : 0.f;
#pragma unroll
                for (int rr = 0; rr < RPW; ++rr) {
                    const float wr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), rr));
#pragma unroll
                    for (int cc2 = 0; cc2 < CPL; ++cc2) oacc[rr][cc2] += acc[rr][cc2] * wr;
                }
                if (lane < RPW && ok16 && a.lse)
                    a.lse[oi16 * 3 + bi] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
            }
        }
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
            for (int cc2 = 0; cc2 < CPL; ++cc2) acc[rr][cc2] = oacc[rr][cc2];
        L = 1.f;                                                     // acc is the output
    } else {
    #pragma unroll
        for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
            for (int cc2 = 0; cc2 < CPL; ++cc2) acc[rr][cc2] = 0.f;
        for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
            uint64_t w[kMergeBatch];
            ovec ov[kMergeBatch][RPW];
#pragma unroll
            for (int i = 0; i < kMergeBatch; ++i) {
                const size_t sp = (size_t)min(s0 + i, S - 1) * RP;
                w[i] = __hip_atomic_load(pml + sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                for (int rr = 0; rr < RPW; ++rr)
                    ov[i][rr] = __hip_atomic_load(pob + (sp + rr) * kWave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            float Mb = M;
#pragma unroll
            for (int i = 0; i < kMergeBatch; ++i) Mb = fmaxf(Mb, __uint_as_float((uint32_t)w[i]));
            if (s0 > 0) {
                // earlier batches: rescale every row by its own factor (lane r's
                // row r; 1 while the row has seen nothing), in every lane
                const float al = (M != -INFINITY && Mb != M) ? __builtin_amdgcn_exp2f(M - Mb) : 1.f;
                L *= al;
#pragma unroll
                for (int rr = 0; rr < RPW; ++rr) {
                    const float alr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), rr));
#pragma unroll
                    for (int cc2 = 0; cc2 < CPL; ++cc2) acc[rr][cc2] *= alr;
                }
            }
            M = Mb;
#pragma unroll
            for (int i = 0; i < kMergeBatch; ++i) {
                if (s0 + i < S) {
                    const float ms = __uint_as_float((uint32_t)w[i]);
                    const float ls = __uint_as_float((uint32_t)(w[i] >> 32));
                    // 0 for an empty split, and for every split of a row no split saw
                    const float sc = M != -INFINITY ? __builtin_amdgcn_exp2f(ms - M) : 0.f;
                    L += ls * sc;
#pragma unroll
                    for (int rr = 0; rr < RPW; ++rr) {
                        const float scr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), rr));
                        if constexpr (CPL == 2) {
                            acc[rr][0] += __uint_as_float((uint32_t)ov[i][rr]) * scr;
                            acc[rr][1] += __uint_as_float((uint32_t)((uint64_t)ov[i][rr] >> 32)) * scr;
                        } else {
                            acc[rr][0] += __uint_as_float((uint32_t)ov[i][rr]) * scr;
                        }
                    }
                }
            }
        }
    }
    const float inv_l = L > 0.f ? 1.f / L : 0.f;                 // lane r16's row
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        const int mr = wave * RPW + rr;
        const int mcq = mr / G, mh = mr - (mr / G) * G;
        if (mcq < Cg && mr < Cg * G) {                           // wave-uniform
            const size_t oi = ((size_t)b * a.NQ + q0 + mcq) * a.H_q + (size_t)g * G + mh;
            const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv_l), rr));
            if constexpr (CPL == 2)
                *reinterpret_cast<float2*>(&a.out[oi * D + lane * 2]) = float2{acc[rr][0] * inv, acc[rr][1] * inv};
            else
                a.out[oi * D + lane] = acc[rr][0] * inv;
        }
    }
    if constexpr (!NSA) {
        bool ok16;
        size_t oi16;
        row16(ok16, oi16);
        if (lane < RPW && ok16 && a.lse) a.lse[oi16] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counters + tg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int D, int RW, bool GRP, bool NSA = false>
hipError_t launch_tw(const TiledArgs& a, hipStream_t s) {
    const size_t lds = tiled_lds_bytes(D, a.bm_words, GRP ? a.nbuf : kPrefillBufs);
    const unsigned tiles = (unsigned)((size_t)a.B * a.H_kv * a.n_tiles * (GRP ? a.n_split : 1));
    hipLaunchKernelGGL((tiled_attn_kernel<D, RW, GRP, NSA>), dim3(tiles), dim3(RW * tiled_ksplit<RW, GRP>() * 64),
                       lds, s, a);
    return hipGetLastError();
}

// verification tiles of RW row waves, plain or three-branch
template <int D>
hipError_t launch_grouped(const TiledArgs& a, int RW, hipStream_t s) {
    if (a.nsa)
        return RW == 8 ? launch_tw<D, 8, true, true>(a, s) : RW == 4 ? launch_tw<D, 4, true, true>(a, s)
             : RW == 2 ? launch_tw<D, 2, true, true>(a, s) : launch_tw<D, 1, true, true>(a, s);
    return RW == 8 ? launch_tw<D, 8, true>(a, s) : RW == 4 ? launch_tw<D, 4, true>(a, s)
         : RW == 2 ? launch_tw<D, 2, true>(a, s) : launch_tw<D, 1, true>(a, s);
}

}  // namespace

// up to 128 rows (32 queries) per tile; waves: the next power of two that
// holds them (2, 4 or 8), padding rows idle
int tiled_queries_per_tile(int G) { return G >= 1 && G <= 32 ? (128 / G < 32 ? 128 / G : 32) : 0; }
int tiled_waves_rows(int rows) {
    const int w = (rows + 15) / 16;
    return w <= 2 ? 2 : (w <= 4 ? 4 : 8);
}
int tiled_waves(int G) { return tiled_waves_rows(tiled_queries_per_tile(G) * G); }
int tiled_grouped_rw(int rows) {
    const int w = (rows + 15) / 16;
    return w <= 1 ? 1 : (w <= 2 ? 2 : (w <= 4 ? 4 : 8));
}

// split-K workspace: [counters, 256-byte padded][(m, l) per split and row][o per split and row]
size_t tiled_ws_bytes(int tiles, int n_split, int waves, int d) {
    if (n_split <= 1) return 0;
    const size_t rows = (size_t)tiles * n_split * waves * 16;
    return ((size_t)tiles * 4 + 255) / 256 * 256 + rows * 2 * 4 + rows * (size_t)d * 4;
}

// slots of K and V, then the bitmap in whole multiples of 16 words
size_t tiled_lds_bytes(int d, int bm_words, int nbuf) {
    return (size_t)nbuf * 2 * kBlock * d * 2 + (size_t)((bm_words + 15) / 16 * 16) * 4;
}

int tiled_grouped_bufs(int d, int bm_words) {
    for (int n = kMaxBufs; n >= 2; --n)
        if (tiled_lds_bytes(d, bm_words, n) <= kTiledLdsMax) return n;
    return 0;
}

hipError_t tiled_grant_lds() {
    const void* kerns[] = {reinterpret_cast<const void*>(tiled_attn_kernel<128, 8, false>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 4, false>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 2, false>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 8, false>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 4, false>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 2, false>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 8, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 4, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 2, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 1, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 8, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 4, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 2, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 1, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 8, true, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 4, true, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 2, true, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<128, 1, true, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 8, true, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 4, true, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 2, true, true>),
                           reinterpret_cast<const void*>(tiled_attn_kernel<64, 1, true, true>)};
    for (const void* k : kerns) {
        const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTiledLdsMax);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// prefill (a.prefill set): kPrefillBufs slots, one workgroup per tile;
// verification: a.nbuf slots (2 .. 4) and a.n_split workgroups per tile, on
// 1, 2, 4 or 8 row waves
hipError_t launch_tiled_attention(const TiledArgs& a, int d, hipStream_t s) {
    const hipError_t e = device_setup();
    if (e != hipSuccess) return e;
    if (a.prefill) {
        const int W = tiled_waves_rows(a.Cq * a.G);
        if (a.n_split != 1 || tiled_lds_bytes(d, a.bm_words, kPrefillBufs) > kTiledLdsMax) return hipErrorInvalidValue;
        if (d == 128) return W == 8 ? launch_tw<128, 8, false>(a, s) : W == 4 ? launch_tw<128, 4, false>(a, s)
                                                                             : launch_tw<128, 2, false>(a, s);
        return W == 8 ? launch_tw<64, 8, false>(a, s) : W == 4 ? launch_tw<64, 4, false>(a, s)
                                                              : launch_tw<64, 2, false>(a, s);
    }
    const int RW = tiled_grouped_rw(a.Cq * a.G);
    if (a.nbuf < 2 || a.nbuf > kMaxBufs || a.n_split < 1 || a.Cq * a.G > 128 || a.Cq > 32 ||
        tiled_lds_bytes(d, a.bm_words, a.nbuf) > kTiledLdsMax)
        return hipErrorInvalidValue;
    // the three-branch mode: a split per branch, and groups of Cu queries that tile Cq
    // groups of Cu queries tile Cq; the three-branch mode needs a split per branch
    if (a.Cu < 1 || a.Cq % a.Cu != 0 || (a.nsa && (a.n_split < 3 || a.cmp_stride < 1)))
        return hipErrorInvalidValue;
    return d == 128 ? launch_grouped<128>(a, RW, s) : launch_grouped<64>(a, RW, s);
}

}  // namespace sda
