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
//       operand, loaded from HBM straight into MFMA layout (16-byte loads,
//       rows past the sequence end clamped, no branches).
//   online softmax per row in fp32 (exp2 with scale*log2(e) folded in).
//   O^T[d][row] += V^T[d][tok] P^T[tok][row]  16x16x32 bf16 MFMA.  V moves
//       HBM -> LDS by direct (DMA) loads, never occupying VGPRs, and is read
//       back transposed with the LDS transpose read; P is split into two
//       bf16 parts (hi + lo, two MFMAs) so about 16 mantissa bits survive,
//       packed from the lane's own scores: the token order inside the QK
//       tile is permuted so each lane already holds the 8 consecutive tokens
//       its PV operand needs.
// HBM-bound: 64*d*2*2 bytes per block and row group; fp32 accumulate.
#include <math.h>
#include <stdlib.h>

#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4i16;
#define SDA_LDS __attribute__((address_space(3)))

// token held in QK A-operand row m of m-tile mt
__device__ __forceinline__ int tok_of(int mt, int m) {
    return (mt >> 1) * 32 + (m >> 2) * 8 + (mt & 1) * 4 + (m & 3);
}

// Wave-private V tile in LDS: 64 rows of d bf16.  The 32-byte chunks of row
// t are XOR-permuted by perm(t) so that the transposed reads (16 rows of one
// logical chunk per instruction) spread over the banks; the direct loads
// write 16-byte pieces in lane order, so each lane fetches the piece that
// belongs at its LDS slot.
template <int D>
struct VTile {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kBytes = kBlock * kRowBytes;
    static constexpr int kLoads = kBytes / (kWave * 16);      // direct loads per lane
    __device__ static __forceinline__ int perm(int t) {
        return D == 128 ? (((t >> 3) & 3) | ((t & 1) << 2)) : ((t >> 3) & 3);
    }
};

template <int D, int NT, int W>
struct SmemPlan {
    static constexpr int RP = NT * 16;
    static constexpr size_t kV = (size_t)W * VTile<D>::kBytes;
    static constexpr size_t kM = (size_t)W * RP * (D + 2) * sizeof(float);
    static constexpr size_t kBase = ((kV > kM ? kV : kM) + 15) / 16 * 16;   // union lists start here
};

// list of blocks a workgroup walks, and which of the group's queries use each
struct ListView {
    const int32_t* gidx;   // global list (C == 1 or shared mode), or null
    const int32_t* lidx;   // LDS list (exact union)
    const uint32_t* lmask; // LDS membership masks (exact union)
    int n;
};

__device__ __forceinline__ void lds_dma16(const void* g, SDA_LDS void* l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

template <int D, int NT, int W>
__device__ __forceinline__ void run_tile_engine(const AttnArgs& a, const ListView& L, int b, int g, int q0,
                                                int Cg, int split, int task, char* smem) {
    constexpr int KS = D / 32;            // QK k-steps
    constexpr int MTD = D / 16;           // PV m-tiles over d
    constexpr int RP = NT * 16;           // padded rows
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int G = a.G;
    const int R = Cg * G;
    const int T = a.seq_len[b];
    const int nb = (T + kBlock - 1) / kBlock;
    const int blocks_cap = (a.T_cap + kBlock - 1) / kBlock;

    // Q fragments (B operand of S^T = K Q^T): row nt*16 + li, d = ks*32 + lg*8
    u32x4 qf[NT][KS];
    int rowq[NT];
    bool rowok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + li;
        const int c = r / G, h = r - c * G;
        rowq[nt] = c;
        rowok[nt] = r < R;
        const uint16_t* qp = a.q + (((size_t)b * a.NQ + q0 + min(c, Cg - 1)) * a.H_q + (size_t)g * G + h) * D + lg * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = ldg16_cached(qp + ks * 32);
            qf[nt][ks] = rowok[nt] ? v : u32x4{0, 0, 0, 0};
        }
    }

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
    const uint16_t* kv_k = a.k + ((size_t)b * a.H_kv + g) * a.T_cap * D;
    const uint16_t* kv_v = a.v + ((size_t)b * a.H_kv + g) * a.T_cap * D;
    // global lists are split over their static width, so a wave's first block
    // id can be read before the row's entry count arrives; entries past the
    // count are padding and skipped
    const int n_range = L.gidx ? a.n_sel_max : L.n;
    const int e_begin = (split * n_range) / a.n_split;
    const int e_end = ((split + 1) * n_range) / a.n_split;
    const int32_t* slot_row = (a.slot && L.gidx) ? a.slot + (L.gidx - a.block_idx) : nullptr;

    // V direct loads: LDS slot (i, lane) holds row i*VRPI + lane/VLPR, 16-byte piece
    // lane % VLPR of the permuted row; the lane fetches the matching logical piece
    constexpr int VLPR = VTile<D>::kRowBytes / 16;         // lanes per V row
    constexpr int VRPI = kWave / VLPR;                      // V rows per direct load
    const int v_lrow = lane / VLPR;
    const int v_rb = (lane % VLPR) * 16;
    const int tr_col = (li & 3) * 8;       // bytes inside the 32-byte chunk for the transposed reads

    auto entry = [&](int e, int& j, int& phys, uint32_t& memb) {
        if (L.gidx) {
            j = L.gidx[e];
            phys = slot_row ? slot_row[e] : j;
            memb = 0xffffffffu;
        } else {
            j = L.lidx[e];
            phys = j;
            memb = L.lmask[e];
        }
    };
    int e = e_begin + wave;
    int j_nx = -1, p_nx = -1;
    uint32_t m_nx = 0;
    if (e < e_end) entry(e, j_nx, p_nx, m_nx);
    for (; e < e_end; e += W) {
        const int j = j_nx, phys = p_nx;
        const uint32_t memb = m_nx;
        if (e + W < e_end) entry(e + W, j_nx, p_nx, m_nx);   // next block id, one iteration early
        if (e >= L.n) break;
        if (j < 0 || j >= nb || phys < 0 || phys >= blocks_cap) continue;
        const int nvalid = min(kBlock, T - j * kBlock);
        if (phys * kBlock + nvalid > a.T_cap) continue;
        const char* kb = reinterpret_cast<const char*>(kv_k + (size_t)phys * kBlock * D);
        const char* vb = reinterpret_cast<const char*>(kv_v + (size_t)phys * kBlock * D);
        const int tmax = nvalid - 1;

        // ---- V into LDS by direct loads, then K into registers (MFMA A layout);
        //      everything is in flight before the first wait ----------------------------
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // previous tile's LDS reads are done
#pragma unroll
        for (int i = 0; i < VTile<D>::kLoads; ++i) {
            const int t = i * VRPI + v_lrow;
            const uint32_t off = (uint32_t)min(t, tmax) * VTile<D>::kRowBytes +
                                 (uint32_t)(v_rb ^ (VTile<D>::perm(t) << 5));
            lds_dma16(vb + off, vs_lds + i * kWave * 16);
        }
        u32x4 kf[4][KS];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const uint32_t off = (uint32_t)min(tok_of(mt, li), tmax) * (D * 2) + lg * 16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kf[mt][ks] = ldg16(kb + off + ks * 64);
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

        // ---- online softmax per row ---------------------------------------------
        u32x4 pf[NT][2], pl[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const bool live = rowok[nt] && ((memb >> rowq[nt]) & 1u);
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = tok_of(mt, lg * 4 + i);
                    float x = s[mt][nt][i] * a.scale_log2;
                    x = (live && t < nvalid) ? x : -INFINITY;
                    s[mt][nt][i] = x;
                    mx = fmaxf(mx, x);
                }
            mx = cross4_max(mx);
            const float m_new = fmaxf(m_run[nt], mx);
            const bool any = m_new != -INFINITY;
            const float m_use = any ? m_new : 0.f;
            const float alpha = any ? __builtin_amdgcn_exp2f(m_run[nt] - m_use) : 1.f;
            float psum = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(s[mt][nt][i] - m_use);   // exp2(-inf) = 0
                    s[mt][nt][i] = p;
                    psum += p;
                }
            psum = cross4_sum(psum);
            l_run[nt] = l_run[nt] * alpha + psum;
            m_run[nt] = m_new;
#pragma unroll
            for (int i = 0; i < MTD; ++i) {
                o[i][nt][0] *= alpha;
                o[i][nt][1] *= alpha;
                o[i][nt][2] *= alpha;
                o[i][nt][3] *= alpha;
            }
            // P^T B operand for token half kh: slot jj = (mt&1)*4 + i with mt = 2*kh + (jj>>2)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float p0 = s[2 * kh + (w >> 1)][nt][(w & 1) * 2];
                    const float p1 = s[2 * kh + (w >> 1)][nt][(w & 1) * 2 + 1];
                    const uint32_t h0 = f2bf(p0), h1 = f2bf(p1);
                    pf[nt][kh][w] = h0 | (h1 << 16);
                    pl[nt][kh][w] = pack_bf16(p0 - __uint_as_float(h0 << 16), p1 - __uint_as_float(h1 << 16));
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

    // ---- merge the waves of this workgroup through LDS -------------------------------
    __syncthreads();
    float* sm_m = reinterpret_cast<float*>(smem);        // [W][RP]
    float* sm_l = sm_m + W * RP;                          // [W][RP]
    float* sm_o = sm_l + W * RP;                          // [W][RP][D]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + li;
        if (lg == 0) {
            sm_m[wave * RP + r] = m_run[nt];
            sm_l[wave * RP + r] = l_run[nt];
        }
#pragma unroll
        for (int md = 0; md < MTD; ++md)
            *reinterpret_cast<floatx4*>(&sm_o[(wave * RP + r) * D + md * 16 + lg * 4]) = o[md][nt];
    }
    __syncthreads();

    const bool final_out = (a.n_split == 1);
    for (int idx = threadIdx.x; idx < R * D; idx += blockDim.x) {
        const int r = idx / D, d = idx - (idx / D) * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w * RP + r]);
        float Ls = 0.f, Os = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float sc = __builtin_amdgcn_exp2f(sm_m[w * RP + r] - M);
                Ls += sm_l[w * RP + r] * sc;
                Os += sm_o[(w * RP + r) * D + d] * sc;
            }
        }
        if (final_out) {
            const int c = r / G, h = r - (r / G) * G;
            const size_t oi = ((size_t)b * a.NQ + q0 + c) * a.H_q + (size_t)g * G + h;
            a.out[oi * D + d] = (Ls > 0.f) ? Os / Ls : 0.f;
            if (d == 0 && a.lse) a.lse[oi] = (Ls > 0.f) ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
        } else {
            const size_t pi = ((size_t)task * a.n_split + split) * RP + r;
            a.part_o[pi * D + d] = Os;
            if (d == 0) {
                a.part_ml[pi * 2] = M;
                a.part_ml[pi * 2 + 1] = Ls;
            }
        }
    }
    if (final_out || !a.fused_combine) return;

    // ---- the last workgroup of this row merges the splits ------------------------------
    int* last = reinterpret_cast<int*>(smem);           // the merge area is free again
    __threadfence();                 // release this split's partials to the other XCDs
    __syncthreads();
    if (threadIdx.x == 0) *last = (atomicAdd(&a.counters[task], 1) == a.n_split - 1);
    __syncthreads();
    if (!*last) return;
    __threadfence();                 // acquire every split's partials
    for (int idx = threadIdx.x; idx < R * D; idx += blockDim.x) {
        const int r = idx / D, d = idx - (idx / D) * D;
        const float* ml = a.part_ml + ((size_t)task * a.n_split * RP + r) * 2;
        const float* po = a.part_o + ((size_t)task * a.n_split * RP + r) * D + d;
        float M = -INFINITY;
        for (int s2 = 0; s2 < a.n_split; ++s2) M = fmaxf(M, __builtin_nontemporal_load(ml + (size_t)s2 * RP * 2));
        float Ls = 0.f, Os = 0.f;
        if (M != -INFINITY) {
            for (int s2 = 0; s2 < a.n_split; ++s2) {
                const float sc = __builtin_amdgcn_exp2f(__builtin_nontemporal_load(ml + (size_t)s2 * RP * 2) - M);
                Ls += __builtin_nontemporal_load(ml + (size_t)s2 * RP * 2 + 1) * sc;
                Os += __builtin_nontemporal_load(po + (size_t)s2 * RP * D) * sc;
            }
        }
        const int c = r / G, h = r - (r / G) * G;
        const size_t oi = ((size_t)b * a.NQ + q0 + c) * a.H_q + (size_t)g * G + h;
        a.out[oi * D + d] = (Ls > 0.f) ? Os / Ls : 0.f;
        if (d == 0 && a.lse) a.lse[oi] = (Ls > 0.f) ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
    }
    if (threadIdx.x == 0) a.counters[task] = 0;          // ready for the next call
}

template <int D, int NT, int W, int MINB>
__global__ __launch_bounds__(W * 64, MINB) void attn_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int task = blockIdx.y;
    const int split = blockIdx.x;
    const int g = task % a.H_kv;
    const int t2 = task / a.H_kv;
    const int grp = t2 % a.n_groups;
    const int b = t2 / a.n_groups;
    const int q0 = grp * a.C;
    const int Cg = min(a.C, a.NQ - q0);
    const int T = a.seq_len[b];
    const int nb = (T + kBlock - 1) / kBlock;

    ListView L{};
    char* after_v = smem + SmemPlan<D, NT, W>::kBase;
    const size_t row0 = ((size_t)b * a.NQ + q0) * a.H_kv + g;   // block_idx row of the group's first query
    if (a.C == 1 || a.mode == 1) {
        L.gidx = a.block_idx + row0 * a.n_sel_max;
        L.n = min(max(a.n_sel[row0], 0), a.n_sel_max);
        if (a.union_count && split == 0 && threadIdx.x == 0 && a.C > 1)
            a.union_count[((size_t)b * a.n_groups + grp) * a.H_kv + g] = L.n;
    } else {
        // exact union of the group's lists: one bitmap per query over the block range
        const int words = (a.NB_cap + 31) / 32;
        uint32_t* bm = reinterpret_cast<uint32_t*>(after_v);               // [C][words]
        int32_t* lidx = reinterpret_cast<int32_t*>(bm + (size_t)a.C * words);
        uint32_t* lmask = reinterpret_cast<uint32_t*>(lidx + (size_t)a.C * a.n_sel_max);
        uint32_t* wsum = lmask + (size_t)a.C * a.n_sel_max;                  // [blockDim.x + 1]
        for (int i = threadIdx.x; i < Cg * words; i += blockDim.x) bm[i] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < Cg * a.n_sel_max; i += blockDim.x) {
            const int c = i / a.n_sel_max, e = i - (i / a.n_sel_max) * a.n_sel_max;
            const size_t rc = row0 + (size_t)c * a.H_kv;
            if (e < a.n_sel[rc]) {
                const int j = a.block_idx[rc * a.n_sel_max + e];
                if (j >= 0 && j < nb && j < a.NB_cap) atomicOr(&bm[c * words + (j >> 5)], 1u << (j & 31));
            }
        }
        __syncthreads();
        // union bits per thread-owned word range, exclusive scan, emit ascending
        const int wpt = (words + blockDim.x - 1) / blockDim.x;
        const int w0 = threadIdx.x * wpt;
        int cnt = 0;
        for (int w = w0; w < min(w0 + wpt, words); ++w) {
            uint32_t u = 0;
            for (int c = 0; c < Cg; ++c) u |= bm[c * words + w];
            cnt += __popc(u);
        }
        wsum[threadIdx.x] = cnt;
        __syncthreads();
        if (threadIdx.x == 0) {
            int run = 0;
            for (int t = 0; t < (int)blockDim.x; ++t) {
                const int v = wsum[t];
                wsum[t] = run;
                run += v;
            }
            wsum[blockDim.x] = run;
        }
        __syncthreads();
        int pos = wsum[threadIdx.x];
        for (int w = w0; w < min(w0 + wpt, words); ++w) {
            uint32_t u = 0;
            for (int c = 0; c < Cg; ++c) u |= bm[c * words + w];
            while (u) {
                const int bit = __ffs(u) - 1;
                u &= u - 1;
                uint32_t mk = 0;
                for (int c = 0; c < Cg; ++c) mk |= ((bm[c * words + w] >> bit) & 1u) << c;
                lidx[pos] = w * 32 + bit;
                lmask[pos] = mk;
                ++pos;
            }
        }
        __syncthreads();
        L.lidx = lidx;
        L.lmask = lmask;
        L.n = wsum[blockDim.x];
        if (a.union_count && split == 0 && threadIdx.x == 0)
            a.union_count[((size_t)b * a.n_groups + grp) * a.H_kv + g] = L.n;
    }
    run_tile_engine<D, NT, W>(a, L, b, g, q0, Cg, split, task, smem);
}

// Split merge as its own launch: one wave per (row group, row); lane s reads
// split s's (m, l), the wave reduces, then each lane merges D/64 columns.
template <int D, int RP>
__global__ __launch_bounds__(64) void combine_kernel(AttnArgs a) {
    const int task = blockIdx.x;
    const int r = blockIdx.y;
    const int g = task % a.H_kv;
    const int t2 = task / a.H_kv;
    const int grp = t2 % a.n_groups;
    const int b = t2 / a.n_groups;
    const int q0 = grp * a.C;
    const int Cg = min(a.C, a.NQ - q0);
    if (r >= Cg * a.G) return;
    const int lane = threadIdx.x;
    const float* ml = a.part_ml + ((size_t)task * a.n_split * RP + r) * 2;
    float M = -INFINITY;
    for (int s2 = lane; s2 < a.n_split; s2 += kWave) M = fmaxf(M, ml[(size_t)s2 * RP * 2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
    constexpr int PER = D / kWave;
    float Os[PER], Ls = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) Os[i] = 0.f;
    if (M != -INFINITY) {
        const float* po = a.part_o + ((size_t)task * a.n_split * RP + r) * D + lane;
#pragma unroll 4
        for (int s2 = 0; s2 < a.n_split; ++s2) {
            const float sc = __builtin_amdgcn_exp2f(ml[(size_t)s2 * RP * 2] - M);
            Ls += ml[(size_t)s2 * RP * 2 + 1] * sc;
#pragma unroll
            for (int i = 0; i < PER; ++i) Os[i] += po[(size_t)s2 * RP * D + i * kWave] * sc;
        }
    }
    const int c = r / a.G, h = r - (r / a.G) * a.G;
    const size_t oi = ((size_t)b * a.NQ + q0 + c) * a.H_q + (size_t)g * a.G + h;
#pragma unroll
    for (int i = 0; i < PER; ++i) a.out[oi * D + lane + i * kWave] = (Ls > 0.f) ? Os[i] / Ls : 0.f;
    if (lane == 0 && a.lse) a.lse[oi] = (Ls > 0.f) ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
}

static int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    return v ? atoi(v) : dflt;
}

int attn_rows_pad(int C, int G) { return (C * G <= 16) ? 16 : 32; }

// workgroup size (waves) of the main decode variant; SDA_ATTN_WAVES overrides (2, 4, 5)
int attn_waves(int d, int rows_pad) {
    if (d == 128 && rows_pad == 16) {
        static const int w = env_int("SDA_ATTN_WAVES", 4);
        return (w == 2 || w == 5) ? w : 4;
    }
    return 4;
}

int attn_default_splits(int list_max, int waves) {
    return (list_max + waves - 1) / waves;      // about one block per wave
}

size_t attn_ws_bytes(int tasks, int n_split, int rows_pad, int d) {
    if (n_split <= 1) return 0;
    const size_t counters = ((size_t)tasks * sizeof(int) + 255) / 256 * 256;
    return counters + (size_t)tasks * n_split * rows_pad * ((size_t)d + 2) * sizeof(float);
}

template <int D, int NT, int W>
static size_t attn_smem_bytes(const AttnArgs& a) {
    size_t extra = 0;
    if (a.C > 1 && a.mode == 0) {
        const size_t words = (size_t)(a.NB_cap + 31) / 32;
        extra = (size_t)a.C * words * 4 + (size_t)a.C * a.n_sel_max * 8 + ((size_t)W * 64 + 1) * 4;
    }
    return SmemPlan<D, NT, W>::kBase + extra;
}

size_t attn_smem_bytes_host(int d, int rows_pad, int C, int mode, int NB_cap, int n_sel_max) {
    const int W = attn_waves(d, rows_pad);
    const size_t vb = (size_t)W * kBlock * d * 2;
    const size_t mb = (size_t)W * rows_pad * (d + 2) * 4;
    size_t base = ((vb > mb ? vb : mb) + 15) / 16 * 16;
    if (C > 1 && mode == 0)
        base += (size_t)C * ((NB_cap + 31) / 32) * 4 + (size_t)C * n_sel_max * 8 + ((size_t)W * 64 + 1) * 4;
    return base;
}

template <int D, int NT, int W, int MINB>
static hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
    const int tasks = a.B * a.n_groups * a.H_kv;
    const size_t smem = attn_smem_bytes<D, NT, W>(a);
    auto kern = attn_kernel<D, NT, W, MINB>;
    static size_t smem_set = 32 * 1024;      // dynamic LDS limit already granted to this variant
    if (smem > smem_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        smem_set = 160 * 1024;
    }
    hipLaunchKernelGGL(kern, dim3(a.n_split, tasks), dim3(W * 64), smem, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1 || a.fused_combine) return e;
    hipLaunchKernelGGL((combine_kernel<D, NT * 16>), dim3(tasks, NT * 16), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a0, hipStream_t s) {
    static const int fused = env_int("SDA_ATTN_FUSED_COMBINE", 0);
    AttnArgs a = a0;
    a.fused_combine = fused;
    const int rp = attn_rows_pad(a.C, a.G);
    if (a.d == 128) {
        if (rp == 16) {
            switch (attn_waves(128, 16)) {
                case 2: return launch_t<128, 1, 2, 3>(a, s);
                case 4: return launch_t<128, 1, 4, 3>(a, s);
                default: return launch_t<128, 1, 5, 3>(a, s);
            }
        }
        return launch_t<128, 2, 4, 1>(a, s);
    }
    if (rp == 16) return launch_t<64, 1, 4, 2>(a, s);
    return launch_t<64, 2, 4, 1>(a, s);
}

}  // namespace sda
