// Block-sparse decode attention and SSV-style grouped verification.
//
// Computes, for every query head, softmax(q K_B^T * scale) V_B over the
// 64-token blocks of its block list ([SparDA] note eq. (7), §4.2 step 4;
// [SSV] note, NSA selection-branch step 3).  The list is split across
// workgroups (split-K); each wave keeps the online-softmax state (m, l, o)
// of the [SSV] note's online-softmax section, waves of a workgroup merge
// through LDS, and a combine pass merges the splits by log-sum-exp.
//
// Grouped mode ([SSV] core mechanism 1, verification-kernel algorithm): a
// workgroup serves the C*G query heads of a group of C consecutive queries
// that share one KV head.  Exact mode walks the union of the C block lists
// (each block read once) and masks every query to its own list; shared mode
// walks the first query's list for all C queries.  Plain decode is the same
// engine with C = 1.
//
// Tile engine (one wave, one 64-token block, rows = the C*G query heads,
// padded to 16 or 32):
//   S^T[tok][row] = K[tok][:] . Q[row][:]   16x16x32 bf16 MFMA, K is the A
//                   operand loaded straight from HBM in MFMA layout (16-byte
//                   loads, four lanes per 64-byte key-row segment);
//   online softmax per row in fp32 (exp2 with scale*log2e folded in);
//   O^T[d][row] += V^T[d][tok] P^T[tok][row]  16x16x32 bf16 MFMA; V goes
//                   HBM -> registers (coalesced rows) -> wave-private LDS and
//                   is read back transposed; P is split into two bf16 parts
//                   (hi + lo, two MFMAs) packed from the lane's own scores:
//                   the token order inside the QK tile is permuted so that
//                   each lane already holds the 8 consecutive tokens its PV
//                   operand needs.
// HBM-bound: 64*d*2*2 bytes per block and row group; fp32 accumulate.
#include <math.h>

#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

constexpr int kWaves = 4;

// token held in QK A-operand row m of m-tile mt (see header comment)
__device__ __forceinline__ int tok_of(int mt, int m) {
    return (mt >> 1) * 32 + (m >> 2) * 8 + (mt & 1) * 4 + (m & 3);
}

// Wave-private V staging: 64 rows of d bf16, unpadded.  The 32-byte chunks of
// row t are XOR-permuted by ((t >> 3) & 3) so that the transposed PV reads
// (four lane groups eight rows apart, sixteen columns each) hit disjoint
// banks while every 16-byte write stays aligned.
template <int D>
struct VStage {
    static constexpr int kBytesPerWave = kBlock * D * 2;
    __device__ static __forceinline__ int col(int t, int c) { return c ^ (((t >> 3) & 3) << 4); }
};

template <int D, int NT>
struct SmemPlan {
    static constexpr int RP = NT * 16;
    static constexpr size_t kV = (size_t)kWaves * VStage<D>::kBytesPerWave;
    static constexpr size_t kM = (size_t)kWaves * RP * (D + 2) * sizeof(float);
    static constexpr size_t kBase = ((kV > kM ? kV : kM) + 15) / 16 * 16;   // union lists start here
};

// list of blocks a workgroup walks, and which of the group's queries use each
struct ListView {
    const int32_t* gidx;   // global list (C == 1 or shared mode), or null
    const int32_t* lidx;   // LDS list (exact union)
    const uint32_t* lmask; // LDS membership masks (exact union)
    int n;
};

template <int D, int NT>
__device__ __forceinline__ void run_tile_engine(const AttnArgs& a, const ListView& L, int b, int g,
                                                int q0, int Cg, int split, int task, char* smem,
                                                float* merge_area) {
    constexpr int KS = D / 32;            // QK k-steps
    constexpr int MTD = D / 16;           // PV m-tiles over d
    constexpr int VLOADS = D / 8;         // 16-byte V loads per lane per block
    constexpr int LPR = D / 8;            // lanes per V row
    constexpr int RPI = kWave / LPR;      // V rows per load instruction
    constexpr int RP = NT * 16;           // padded rows
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int G = a.G;
    const int R = Cg * G;
    const int T = a.seq_len[b];
    const int nb = (T + kBlock - 1) / kBlock;
    const int blocks_cap = a.T_cap / kBlock + ((a.T_cap % kBlock) ? 1 : 0);

    // Q fragments (B operand of S^T = K Q^T): row nt*16 + li, d = ks*32 + lg*8
    u32x4 qf[NT][KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + li;
        const int c = r / G, h = r - (r / G) * G;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (r < R) {
                const size_t qo = (((size_t)b * a.NQ + q0 + c) * a.H_q + (size_t)g * G + h) * D + ks * 32 + lg * 8;
                qf[nt][ks] = ldg16_cached(a.q + qo);
            } else {
                qf[nt][ks] = u32x4{0, 0, 0, 0};
            }
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
    // which group query owns this lane's row, per n-tile (for masking)
    int rowq[NT];
    bool rowok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + li;
        rowq[nt] = r / G;
        rowok[nt] = r < R;
    }

    uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + (size_t)wave * kBlock * D;
    const size_t kv_row = ((size_t)b * a.H_kv + g) * a.T_cap;   // first token of this (b, g) buffer
    const int e_begin = (int)(((long long)split * L.n) / a.n_split);
    const int e_end = (int)(((long long)(split + 1) * L.n) / a.n_split);

    for (int e = e_begin + wave; e < e_end; e += kWaves) {
        int j;
        uint32_t memb = 0xffffffffu;
        if (L.gidx) {
            j = L.gidx[e];
        } else {
            j = L.lidx[e];
            memb = L.lmask[e];
        }
        int phys = j;
        if (a.slot && L.gidx) phys = a.slot[(L.gidx - a.block_idx) + e];
        if (j < 0 || j >= nb || phys < 0 || phys >= blocks_cap) continue;
        const int nvalid = min(kBlock, T - j * kBlock);
        if (phys * kBlock + nvalid > a.T_cap) continue;
        const uint16_t* kb = a.k + (kv_row + (size_t)phys * kBlock) * D;
        const uint16_t* vb = a.v + (kv_row + (size_t)phys * kBlock) * D;

        // ---- loads: K in MFMA A layout, V in row order ------------------------
        u32x4 kf[4][KS];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int t = tok_of(mt, li);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (t < nvalid) kf[mt][ks] = ldg16(kb + (size_t)t * D + ks * 32 + lg * 8);
                else kf[mt][ks] = u32x4{0, 0, 0, 0};
            }
        }
        u32x4 vr[VLOADS];
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int t = i * RPI + lane / LPR;
            if (t < nvalid) vr[i] = ldg16(vb + (size_t)t * D + (lane % LPR) * 8);
            else vr[i] = u32x4{0, 0, 0, 0};
        }

        // ---- S^T = K Q^T ------------------------------------------------------
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

        // ---- stage V (wave-private LDS) ---------------------------------------
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
            const int t = i * RPI + lane / LPR;
            *reinterpret_cast<u32x4*>(vs + t * D + VStage<D>::col(t, (lane % LPR) * 8)) = vr[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

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
            float alpha = 1.f;
            float psum = 0.f;
            if (m_new != -INFINITY) {
                alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float p = __builtin_amdgcn_exp2f(s[mt][nt][i] - m_new);
                        s[mt][nt][i] = p;
                        psum += p;
                    }
            } else {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[mt][nt][i] = 0.f;
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
            // P^T B operand for token half kh: slots j = (mt&1)*4 + i with mt = 2*kh + (j>>2).
            // P = hi + lo with both parts bf16, so V^T P^T keeps ~16 mantissa bits of P
            // and the result does not depend on where the running maximum stood.
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

        // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            // rows kh*32 + lg*8 + 0..7 all carry chunk permutation lg
            const uint16_t* vrow = vs + (kh * 32 + lg * 8) * D + li;
#pragma unroll
            for (int md = 0; md < MTD; ++md) {
                const uint16_t* p = vrow + ((md ^ lg) << 4);
                u32x4 va;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t lo = p[(2 * w) * D];
                    const uint32_t hi = p[(2 * w + 1) * D];
                    va[w] = lo | (hi << 16);
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    o[md][nt] = mfma16x16x32(va, pf[nt][kh], o[md][nt]);
                    o[md][nt] = mfma16x16x32(va, pl[nt][kh], o[md][nt]);
                }
            }
        }
    }

    // ---- merge the waves of this workgroup through LDS ---------------------------
    __syncthreads();
    float* sm_m = merge_area;                            // [kWaves][RP]
    float* sm_l = sm_m + kWaves * RP;                    // [kWaves][RP]
    float* sm_o = sm_l + kWaves * RP;                    // [kWaves][RP][D]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + li;
        if (lg == 0) {
            sm_m[wave * RP + r] = m_run[nt];
            sm_l[wave * RP + r] = l_run[nt];
        }
#pragma unroll
        for (int md = 0; md < MTD; ++md)
#pragma unroll
            for (int i = 0; i < 4; ++i) sm_o[((size_t)wave * RP + r) * D + md * 16 + lg * 4 + i] = o[md][nt][i];
    }
    __syncthreads();

    const bool final_out = (a.n_split == 1);
    for (int idx = threadIdx.x; idx < R * D; idx += blockDim.x) {
        const int r = idx / D, d = idx - (idx / D) * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * RP + r]);
        float Ls = 0.f, Os = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float sc = __builtin_amdgcn_exp2f(sm_m[w * RP + r] - M);
                Ls += sm_l[w * RP + r] * sc;
                Os += sm_o[((size_t)w * RP + r) * D + d] * sc;
            }
        }
        const int c = r / G, h = r - (r / G) * G;
        if (final_out) {
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
}

template <int D, int NT, int MINB>
__global__ __launch_bounds__(256, MINB) void attn_kernel(AttnArgs a) {
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
    char* after_v = smem + SmemPlan<D, NT>::kBase;
    const size_t row0 = ((size_t)b * a.NQ + q0) * a.H_kv + g;   // block_idx row of the group's first query
    if (a.C == 1 || a.mode == 1) {
        L.gidx = a.block_idx + row0 * a.n_sel_max;
        L.n = min(max(a.n_sel[row0], 0), a.n_sel_max);
        if (a.union_count && split == 0 && threadIdx.x == 0 && a.C > 1)
            a.union_count[((size_t)b * a.n_groups + grp) * a.H_kv + g] = L.n;
    } else {
        // exact union of the group's lists: one bitmap per query over the block range
        const int words = (a.NB_cap + 31) / 32;
        uint32_t* bm = reinterpret_cast<uint32_t*>(after_v);               // [Cg][words]
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
        // count union bits per thread-owned word range, exclusive scan, emit ascending
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
    run_tile_engine<D, NT>(a, L, b, g, q0, Cg, split, task, smem, reinterpret_cast<float*>(smem));
}

// merge the splits of each (task, row) by log-sum-exp
template <int D, int RP>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
    const int task = blockIdx.x;
    const int g = task % a.H_kv;
    const int t2 = task / a.H_kv;
    const int grp = t2 % a.n_groups;
    const int b = t2 / a.n_groups;
    const int q0 = grp * a.C;
    const int Cg = min(a.C, a.NQ - q0);
    const int R = Cg * a.G;
    for (int idx = threadIdx.x; idx < R * D; idx += blockDim.x) {
        const int r = idx / D, d = idx - (idx / D) * D;
        float M = -INFINITY;
        for (int s = 0; s < a.n_split; ++s)
            M = fmaxf(M, a.part_ml[(((size_t)task * a.n_split + s) * RP + r) * 2]);
        float Ls = 0.f, Os = 0.f;
        if (M != -INFINITY) {
            for (int s = 0; s < a.n_split; ++s) {
                const size_t pi = ((size_t)task * a.n_split + s) * RP + r;
                const float sc = __builtin_amdgcn_exp2f(a.part_ml[pi * 2] - M);
                Ls += a.part_ml[pi * 2 + 1] * sc;
                Os += a.part_o[pi * D + d] * sc;
            }
        }
        const int c = r / a.G, h = r - (r / a.G) * a.G;
        const size_t oi = ((size_t)b * a.NQ + q0 + c) * a.H_q + (size_t)g * a.G + h;
        a.out[oi * D + d] = (Ls > 0.f) ? Os / Ls : 0.f;
        if (d == 0 && a.lse) a.lse[oi] = (Ls > 0.f) ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
    }
}

int attn_rows_pad(int C, int G) { return (C * G <= 16) ? 16 : 32; }

int attn_default_splits(int list_max) {
    const int per_wg = kWaves;   // one block per wave
    return (list_max + per_wg - 1) / per_wg;
}

size_t attn_ws_bytes(int tasks, int n_split, int rows_pad, int d) {
    if (n_split <= 1) return 0;
    return (size_t)tasks * n_split * rows_pad * ((size_t)d + 2) * sizeof(float);
}

template <int D, int NT>
static size_t attn_smem_bytes(const AttnArgs& a) {
    size_t extra = 0;
    if (a.C > 1 && a.mode == 0) {
        const size_t words = (size_t)(a.NB_cap + 31) / 32;
        extra = (size_t)a.C * words * 4 + (size_t)a.C * a.n_sel_max * 8 + (256 + 1) * 4;
    }
    return SmemPlan<D, NT>::kBase + extra;
}

template <int D, int NT, int MINB>
static hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
    const int tasks = a.B * a.n_groups * a.H_kv;
    const size_t smem = attn_smem_bytes<D, NT>(a);
    auto kern = attn_kernel<D, NT, MINB>;
    if (smem > 32 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(a.n_split, tasks), dim3(256), smem, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    hipLaunchKernelGGL((combine_kernel<D, NT * 16>), dim3(tasks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    const int rp = attn_rows_pad(a.C, a.G);
    if (a.d == 128) {
        if (rp == 16) return launch_t<128, 1, 2>(a, s);
        return launch_t<128, 2, 1>(a, s);
    }
    if (rp == 16) return launch_t<64, 1, 2>(a, s);
    return launch_t<64, 2, 1>(a, s);
}

}  // namespace sda
