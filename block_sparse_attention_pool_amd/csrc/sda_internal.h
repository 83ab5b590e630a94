// Internal host-side declarations shared by the C-ABI layer and the kernel
// translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sda {

// ---- compressed keys ----------------------------------------------------------
// entry j of a row: mean of tokens [j*stride, min(j*stride + window, len)), window <= 64
hipError_t launch_update_compressed_keys(const uint16_t* k, uint16_t* kt, const int32_t* len_old,
                                         const int32_t* len_new, int max_entries_per_row, int B,
                                         int H_kv, int d, int T_cap, int NC_cap, int window, int stride,
                                         hipStream_t s);

// ---- scoring and selection ----------------------------------------------------
struct SelectArgs {
    const int32_t* seq_len;
    const float* scores;     // [rows, NB_cap]
    int rows, NQ, H_kv, NB_cap;
    int n_init, n_local, top_k, n_sel_max;
    int32_t* block_idx;
    int32_t* n_sel;
};
// scores, then exact top-k and block sets.  With `cand` and `counters` (zeroed,
// one per (b, kv head, vector tile)) the selection runs inside the scoring
// launch (needs fused_select_ok); otherwise scores go to scores_opt or
// scores_ws and a second launch selects.
hipError_t launch_score_select(const uint16_t* f, const uint16_t* kt, const SelectArgs& sel, int B, int d,
                               float* scores_opt, float* scores_ws, uint64_t* cand, int* counters,
                               hipStream_t s);
bool fused_select_ok(int NB_cap, int top_k);
// overlapping compression: entries of kernel `window`, stride `stride`
// (NC_cap per row) scored, max-pooled onto the 64-token blocks (sel.NB_cap
// per row), then selected as launch_score_select does
hipError_t launch_score_select_pooled(const uint16_t* f, const uint16_t* kt, const SelectArgs& sel, int B, int d,
                                      int window, int stride, int NC_cap, float* scores_opt, float* scores_ws,
                                      uint64_t* cand, int* counters, hipStream_t s);

constexpr int kFusedTopK = 64;       // longest per-chunk list the in-launch selection keeps
constexpr int kFusedChunks = 16;     // most 256-block chunks it merges (NB_cap <= 4096)
// top-k lists are padded to the smallest power of two >= K (1 for K = 0)
__host__ __device__ inline int pow2_at_least(int K) {
    int P = 1;
    while (P < K) P <<= 1;
    return P;
}
// LDS of the decode step's scoring workgroups: per group of four waves the
// chunk's scores and four sorted wave lists, then the level-2 buffers and
// one flag per group
__host__ __device__ inline size_t step_group_lds_bytes(int K) {
    (void)K;
    return 256 * 4 + 4 * 64 * 8;
}
__host__ __device__ inline size_t step_lds_bytes(int K, int cpr, int per_wg) {
    const size_t P = (size_t)pow2_at_least(K);
    return per_wg * step_group_lds_bytes(K) + (P * cpr + P * ((cpr + 1) / 2)) * 8 + 16;
}
int score_tiles(int NQ, int NB_cap, int rows);            // vector tiles of the scoring grid
int score_tile_vectors(int nvec, int NB_cap, int rows);    // vectors per scoring workgroup
// G-head comparator: scores plus per-chunk softmax statistics, then per-block
// sums of the heads' softmax weights and the selection (inside the second
// launch when cand / counters are given, else a third launch)
hipError_t launch_multihead_select(const uint16_t* q, const uint16_t* kt, const SelectArgs& sel, int B, int H_q,
                                   int d, float tau, float* z, float* stats, float* scores_opt, float* scores_ws,
                                   uint64_t* cand, int* counters, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
// the G-head comparator on overlapping compressed entries (kernel `window`,
// stride `stride`, NC_cap per row), max-pooled onto the 64-token blocks
hipError_t launch_multihead_select_pooled(const uint16_t* q, const uint16_t* kt, const SelectArgs& sel, int B,
                                          int H_q, int d, float tau, int window, int stride, int NC_cap, float* z,
                                          float* stats, float* scores_opt, float* scores_ws, uint64_t* cand,
                                          int* counters, hipStream_t s);
size_t multihead_ws_floats(int B, int NQ, int H_q, int H_kv, int NB_cap);
int score_chunks(int NB_cap);

// ---- prefill selection ----------------------------------------------------------
// query r of a chunk sits at position pos0 + r; its block scores live in
// registers, so the blocks a query sees are bounded (positions < 64 * 512)
constexpr int kPrefillMaxBlocks = 512;
struct PrefillSelectArgs {
    const uint16_t* f;        // [B, NQ, H_kv, d] indexer vectors
    const uint16_t* kt;       // [B, H_kv, NB_cap, d] compressed keys
    const int32_t* seq_len;   // [B] cached tokens; queries at positions >= seq_len get no blocks
    int B, NQ, H_kv, NB_cap, pos0;
    int n_init, n_local, top_k, n_sel_max;
    int32_t* block_idx;       // [B, NQ, H_kv, n_sel_max]
    int32_t* n_sel;           // [B, NQ, H_kv]
};
hipError_t launch_prefill_select(const PrefillSelectArgs& a, int d, hipStream_t s);

constexpr int kCUs = 256;                  // MI355X compute units

// ---- attention ------------------------------------------------------------------
// The next layer's scoring and selection inside a decode launch: each extra
// workgroup scores per_wg 256-block chunks (one per group of four waves) and
// keeps each chunk's top-k keys; the last workgroup to finish a row's chunks
// merges them into the row's block set.
struct StepScore {
    const uint16_t* vec;      // next layer's indexer vectors, bf16 [rows, D] (NQ = 1)
    const uint16_t* kt;       // next layer's compressed keys, bf16 [rows, NB_cap, D]
    uint64_t* cand;           // [rows, cpr, top_k] per-chunk lists
    int* counters;            // [rows] chunk arrivals; zero between calls
    SelectArgs sel;           // rows = B * H_kv
    int cpr;                  // chunks per row
    int per_wg;               // chunks per workgroup pass (groups of four waves)
    int passes;               // passes per scoring workgroup (chunks w * passes * per_wg ..)
    // Optional: workgroups after the scoring ones refresh this layer's
    // compressed keys for the tokens [ref_len_old, seq_len) (ref_kt null = off)
    uint16_t* ref_kt;         // [B, H_kv, ref_NB_cap, D]
    const int32_t* ref_len_old;
    int ref_NB_cap;
    int ref_blocks;           // blocks refreshed per row (grid bound)
    int ref_rows;             // grid rows of refresh workgroups after the scoring ones (set at launch)
};
struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* seq_len;
    const int32_t* block_idx;
    const int32_t* n_sel;
    const int32_t* slot;      // may be null
    float* out;
    float* lse;               // may be null
    int32_t* union_count;     // may be null
    float* part_o;            // [tasks, n_split, rows_pad, d]
    float* part_ml;           // [tasks, n_split, rows_pad, 2]
    int* counters;            // [tasks] split arrivals; zero between calls
    int n_sel_max, T_cap, NB_cap;
    int B, NQ, H_q, H_kv, G, d;
    int C;                    // queries per group (1 = plain decode)
    int mode;                 // 0 exact, 1 shared representative
    int n_groups;             // ceil(NQ / C)
    int task0;                // first row group of this launch (launches cover at most 65535)
    int n_split;
    int waves;                // waves per workgroup
    float scale_log2;         // scale * log2(e)
    // Optional (the decode-step entry point): workgroups past the attention
    // grid score the next layer and select its blocks (step.cand null = off)
    StepScore step;
    // NSA three-branch mode (nsa = 1): splits [0, ns_c) attend to the
    // compressed cache, [ns_c, ns_c + ns_s) to the listed blocks, the rest to
    // the last `window` tokens; the last workgroup of a row group merges each
    // branch's splits and writes the gated sum
    int nsa;
    const uint16_t* kc;       // compressed keys   [B, H_kv, NC_cap, d]
    const uint16_t* vc;       // compressed values [B, H_kv, NC_cap, d]
    const float* gates;       // [B, NQ, H_q, 3]: g_c, g_s, g_w
    int NC_cap, cmp_stride, window;
    int ns_c, ns_s;
};
struct AttnPlan {
    int waves;                // waves per workgroup
    int n_split;              // workgroups per row group
};
int attn_rows_pad(int C, int G);                 // 16 or 32
AttnPlan attn_plan(int d, int rows_pad, int tasks, int list_max, int C, int mode, int NB_cap, int n_sel_max,
                   int split_k);
size_t attn_ws_bytes(int tasks, int n_split, int rows_pad, int d);
size_t attn_smem_bytes_host(int d, int rows_pad, int W, int C, int mode, int NB_cap, int n_sel_max);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// gives every attention kernel the compute unit's whole LDS (160 KB) on the
// current device; called once per device by device_setup()
hipError_t attn_grant_lds();

// ---- row-tiled attention (prefill) --------------------------------------------------
// A workgroup holds up to 128 rows (Cq queries x G heads) of one (b, g) and
// walks the union of their block lists through LDS (two blocks in flight, so
// that two workgroups share a compute unit); see k_tiled.hip.
constexpr size_t kTiledLdsMax = 160 * 1024;
struct TiledArgs {
    const uint16_t* q;        // [B, NQ, H_q, d]
    const uint16_t* k;        // [B, H_kv, T_cap, d]
    const uint16_t* v;
    const int32_t* seq_len;   // [B]
    const int32_t* block_idx; // [B, NQ, H_kv, n_sel_max] ascending
    const int32_t* n_sel;     // [B, NQ, H_kv]
    float* out;               // [B, NQ, H_q, d]
    float* lse;               // [B, NQ, H_q] or null
    int n_sel_max, T_cap, NB_cap;
    int B, NQ, H_q, H_kv, G;
    int Cq;                   // queries per tile
    int n_tiles;              // ceil(NQ / Cq)
    int prefill, pos0;        // prefill: query q sees tokens below pos0 + q + 1
    int bm_words;             // bitmap words in LDS: >= the blocks any tile may list
    int nbuf;                 // verification tiles: K/V slots in LDS (2 .. 4); prefill uses 2
    float scale_log2;
    // split-K (n_split > 1): the union of a tile is shared among n_split
    // workgroups; each writes (m, l, o) of its rows and the last to arrive merges
    int n_split;
    float* part_o;            // [tiles, n_split, 16 W, d]
    float* part_ml;           // [tiles, n_split, 16 W, 2]
    int* counters;            // [tiles]; zero between calls
    int32_t* union_count;     // [B, n_ugroups, H_kv] blocks in each group's union, or null
    int Cu, n_ugroups;        // verification: groups of Cu queries (Cu divides Cq), ceil(NQ / Cu)
    int rep;                  // verification: every query takes its group's first list (shared mode)
    // NSA three-branch mode (nsa = 1, verification tiles only): every tile
    // splits its n_split workgroups among the compressed cache, its listed
    // blocks and the window in proportion to their block counts (computed
    // alike by every workgroup of the tile); the last to arrive merges each
    // branch and writes the gated sum and the three lse.
    int nsa;
    const uint16_t* kc;       // compressed keys   [B, H_kv, NC_cap, d]
    const uint16_t* vc;       // compressed values [B, H_kv, NC_cap, d]
    const float* gates;       // [B, NQ, H_q, 3]: g_c, g_s, g_w
    int NC_cap, cmp_stride, window;
};
int tiled_queries_per_tile(int G);
int tiled_waves_rows(int rows);   // 2, 4 or 8 waves for up to 128 rows
int tiled_waves(int G);
int tiled_grouped_rw(int rows);   // verification tiles: 1, 2, 4 or 8 row waves for up to 128 rows
size_t tiled_ws_bytes(int tiles, int n_split, int waves, int d);
size_t tiled_lds_bytes(int d, int bm_words, int nbuf);
int tiled_grouped_bufs(int d, int bm_words);   // most slots (<= 4) that fit beside the bitmap; 0 if none
hipError_t tiled_grant_lds();
hipError_t launch_tiled_attention(const TiledArgs& a, int d, hipStream_t s);

// ---- per-device set-up ----------------------------------------------------------------
// Done once per device, at the first call of any entry point on it, under a
// lock: grants the attention kernels their LDS.  The record never changes
// after it is written and never changes results.
hipError_t device_setup();

// The no-allocation decode step's scratch: a static device array of
// kNoallocScratchBytes per device, its first kNoallocCounterBytes reserved
// for arrival counters.  noalloc_scratch() returns its device address on the
// current device (looked up once per device; the first lookup also clears
// the counter region with a fill kernel on stream s).
constexpr size_t kNoallocScratchBytes = (size_t)8 << 20;
constexpr size_t kNoallocCounterBytes = (size_t)64 << 10;
hipError_t noalloc_scratch(hipStream_t s, char** ptr);

// ---- offload gather -----------------------------------------------------------------
hipError_t launch_gather(const uint16_t* k_src, const uint16_t* v_src, const int32_t* block_idx,
                         const int32_t* n_sel, int n_sel_max, int B, int H_kv, int d, int T_cap,
                         uint16_t* k_stage, uint16_t* v_stage, int32_t* slot_out,
                         int max_workgroups, hipStream_t s);

// ---- persistent prefetch pool (offloaded K/V chain) -------------------------------
constexpr int kMaxChainLayers = 32;
constexpr int kPfTail = 0, kPfStop = 1, kPfError = 2, kPfClaim = 8, kPfDone = 8 + kMaxChainLayers;
constexpr int kPfCtrlInts = 8 + 2 * kMaxChainLayers;
struct PrefetchLayer {
    const uint16_t* k_src;    // device-mapped pinned host K [B, H_kv, T_cap, d]
    const uint16_t* v_src;
    const int32_t* block_idx; // [B, 1, H_kv, n_sel_max] the layer's block lists
    const int32_t* n_sel;     // [B, 1, H_kv]
    uint16_t* k_stage;        // [B, H_kv, n_sel_max * 64, d]
    uint16_t* v_stage;
    int32_t* slot;            // [B, 1, H_kv, n_sel_max]
};
struct PrefetchArgs {
    PrefetchLayer layer[kMaxChainLayers];
    int L, rows, n_sel_max, T_cap;
    int* ctrl;                // kPfCtrlInts control words
    int spin_limit;           // polls before a wait gives up
};
hipError_t launch_prefetch_reset(int* ctrl, hipStream_t s);
hipError_t launch_zero_words(void* p, size_t bytes, hipStream_t s);       // fill kernel: bytes / 4 zero words
hipError_t launch_prefetch_pool(const PrefetchArgs& a, int d, int workgroups, hipStream_t s);
hipError_t launch_prefetch_enqueue(int* ctrl, int r, hipStream_t s);
hipError_t launch_prefetch_wait(int* ctrl, int r, int total, int spin_limit, hipStream_t s);
hipError_t launch_prefetch_stop(int* ctrl, hipStream_t s);

}  // namespace sda
