/*
 * sda.h - top-k block-sparse decode attention on MI355X (gfx950).
 *
 * C ABI of libsda.so.  Every call validates its arguments on the host before
 * anything is enqueued; on a validation error nothing is launched and a
 * non-zero status is returned (details in sda_last_error()).  Calls are
 * asynchronous on `stream` (a hipStream_t; NULL = the default stream) and
 * never synchronise the host.  The library allocates no memory: callers pass
 * device buffers and a workspace sized by the matching *_workspace() call.
 * All pointers are device pointers unless the comment says "host".
 * Tensors are dense, row-major, in the shapes given in brackets.
 *
 * Sources (by page title, section and equation):
 *   [SparDA] reading note "SparDA：稀疏解耦注意力，让长上下文推理又快又准"
 *            (zhongzhuzhou.org, 2026-06-24), on SparDA: Sparse Decoupled
 *            Attention (arXiv 2606.04511).
 *   [SSV]    reading note "SSV：稀疏投机验证——在动态稀疏注意力中做投机解码"
 *            (zhongzhuzhou.org, 2026-07-01), on SSV (arXiv 2605.19893).
 *
 * Shapes and symbols: B batch, NQ queries per sequence (1 for plain decode),
 * H_q query heads, H_kv KV heads, G = H_q / H_kv, d head dim (64 or 128),
 * T_cap token capacity of the K/V buffers, NB_cap = block capacity of the
 * compressed-key buffer (>= ceil(T_cap / 64)).  Blocks are 64 tokens.  Query
 * head h uses KV head h / G.  bf16 tensors are passed as raw 16-bit storage.
 * A "row" is one (batch, query, KV head).
 */
#ifndef SDA_H
#define SDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SDA_OK = 0,
    SDA_ERR_NULL = 1,        /* a required pointer is NULL */
    SDA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes */
    SDA_ERR_UNSUPPORTED = 3, /* valid request outside what the kernels cover (e.g. d = 96) */
    SDA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than *_workspace() asks */
    SDA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
    SDA_ERR_HIP = 6          /* the HIP runtime reported an error (launch or query) */
} sda_status_t;

enum { SDA_GROUP_EXACT = 0, SDA_GROUP_SHARED_REP = 1 };

#define SDA_BLOCK_TOKENS 64

/* Name of a status code (static string). */
const char* sda_status_string(sda_status_t s);

/* Detail of the last error returned on the calling thread (thread-local,
 * valid until the next failing call on that thread; "" when none). */
const char* sda_last_error(void);

/* Library version string, e.g. "sda 0.1 gfx950". */
const char* sda_version(void);

/*
 * Compressed keys: K~[b,g,j,:] = mean of K[b,g,64j : min(64j+64, len), :]
 * ([SparDA] prerequisites §3, eq. (4) with kernel = stride = 64; kept on the
 * GPU and refreshed as tokens are appended, §4.2 step 1 and §4.6), stored in
 * bf16 like the keys: the mean is formed in fp64 (exact sums of bf16 values
 * whenever a block's non-zero magnitudes lie within a factor 2^39) and
 * rounded once to the nearest bf16, ties to even.
 *
 *   k        bf16 [B, H_kv, T_cap, d]        keys (read only)
 *   k_tilde  bf16 [B, H_kv, NB_cap, d]       updated in place
 *   len_old  i32  [B]  tokens already pooled; len_new i32 [B] tokens now cached
 *
 * Every block touched by tokens [len_old[b], len_new[b]) is recomputed from
 * K (the whole block, so an incremental update equals a bulk build bit for
 * bit).  Bulk build: len_old = 0, len_new = T.  max_new_tokens must bound
 * len_new[b] - len_old[b] for every b (it sizes the grid; rows needing more
 * are truncated).  Device-side guards: len_new is clamped to T_cap and rows
 * with len_new <= len_old are left unchanged.
 */
sda_status_t sda_update_compressed_keys(const void* k, void* k_tilde,
                                        const int32_t* len_old, const int32_t* len_new,
                                        int max_new_tokens, int B, int H_kv, int d,
                                        int T_cap, int NB_cap, void* stream);

/*
 * Indexer scoring, top-k and block-set assembly for every row
 * ([SparDA] §4.2 step 2, eq. (3), (6), (9); [SSV] NSA selection branch
 * steps 1-2):
 *   s_j = f . K~_j for each of the row's nb = ceil(seq_len[b] / 64) blocks;
 *   B = {0..n_init-1} U {nb-n_local..nb-1} U top_k(s over the other blocks),
 *   ties to the lower block index; written ascending, padded with -1.
 * f is one indexer (Forecast) vector per row; with SparDA's lookahead it is
 * layer l's vector scored against layer l+1's compressed keys (eq. (6)).
 *
 *   f          bf16 [B, NQ, H_kv, d]
 *   k_tilde    bf16 [B, H_kv, NB_cap, d]
 *   seq_len    i32  [B]               (1 <= seq_len <= 64 * NB_cap)
 *   block_idx  i32  [B, NQ, H_kv, n_sel_max] out; n_sel i32 [B, NQ, H_kv] out
 *   scores_opt f32  [B, NQ, H_kv, NB_cap] out or NULL (raw scores, entries past nb undefined)
 * n_sel_max >= n_init + n_local + top_k.  Scores are fp32 sums of the exact
 * bf16 x bf16 products.
 * Workspace: sda_score_select_workspace() bytes, required even with scores_opt.
 * It holds arrival counters: zero-fill it before its first use; every
 * completed call leaves them zero.  Calls sharing a workspace must not overlap
 * in time.  With top_k <= 64 and NB_cap <= 4096 the selection runs inside the
 * scoring launch, otherwise as a second launch; the results are identical.
 */
size_t sda_score_select_workspace(int B, int NQ, int H_kv, int NB_cap, int top_k);
sda_status_t sda_score_select(const void* f, const void* k_tilde, const int32_t* seq_len,
                              int B, int NQ, int H_kv, int d, int NB_cap,
                              int n_init, int n_local, int top_k, int n_sel_max,
                              int32_t* block_idx, int32_t* n_sel, float* scores_opt,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * G-head block selector used as the comparator to the one-head indexer
 * ([SparDA] §4.3 eq. (8) and the target of §4.4 eq. (10)): for each row,
 * s_j = sum over the G query heads h of the row's KV group of
 * softmax over all nb blocks of (q_h . K~_j / tau); then the same top-k and
 * block-set assembly as sda_score_select.  With 64-token pooling windows the
 * max-pool onto the block grid is the identity.
 *
 *   q  bf16 [B, NQ, H_q, d]; other arguments as sda_score_select; tau > 0.
 * Workspace: sda_score_select_multihead_workspace() bytes.
 */
size_t sda_score_select_multihead_workspace(int B, int NQ, int H_q, int H_kv, int NB_cap, int top_k);
sda_status_t sda_score_select_multihead(const void* q, const void* k_tilde, const int32_t* seq_len,
                                        int B, int NQ, int H_q, int H_kv, int d, int NB_cap,
                                        int n_init, int n_local, int top_k, int n_sel_max, float tau,
                                        int32_t* block_idx, int32_t* n_sel, float* scores_opt,
                                        void* ws, size_t ws_bytes, void* stream);

/*
 * InfLLM-V2's block selector on overlapping compressed keys, the setting of
 * the pages' selection-cost comparison ([SparDA] §4.3 eq. (8) and fig. 3:
 * the G query heads of the KV group score every compressed key, each head's
 * scores pass through a softmax over all entries, the G softmaxes are summed,
 * and the sums are max-pooled onto the 64-token block grid; §4.4: kernel
 * l = 32, stride s = 16 at inference): for each row,
 *   s_e = sum_h softmax_e(q_h . K~_e / tau) over the ceil(seq_len / s) entries;
 *   S_J = max of s_e over the windows that share a token with block J;
 *   then init, local and top-k as sda_score_select.
 * Arguments as sda_score_select_multihead, with k_tilde from
 * sda_update_compressed_keys_strided ([B, H_kv, NC_cap, d]) and window /
 * stride as sda_score_select_pooled; scores_opt [B, NQ, H_kv,
 * ceil(NC_cap * stride / 64)] or NULL.  Workspace:
 * sda_score_select_multihead_pooled_workspace() bytes, zero-filled before
 * first use.
 */
size_t sda_score_select_multihead_pooled_workspace(int B, int NQ, int H_q, int H_kv, int NC_cap, int stride,
                                                   int top_k);
sda_status_t sda_score_select_multihead_pooled(const void* q, const void* k_tilde, const int32_t* seq_len, int B,
                                               int NQ, int H_q, int H_kv, int d, int NC_cap, int window, int stride,
                                               int n_init, int n_local, int top_k, int n_sel_max, float tau,
                                               int32_t* block_idx, int32_t* n_sel, float* scores_opt, void* ws,
                                               size_t ws_bytes, void* stream);

/*
 * Overlapping compressed keys ([SparDA] prerequisites §3, eq. (4) with kernel
 * l = window and stride s = stride; §4.4 quotes InfLLM-V2's inference setting
 * l = 32, s = 16): entry j of a row is the mean of the keys
 * K[b,g, j*s : min(j*s + l, len), :] for every j with j*s < len, rounded once
 * to bf16 as in sda_update_compressed_keys (whose 64/64 case this is).
 *
 *   k        bf16 [B, H_kv, T_cap, d]        keys (read only)
 *   k_tilde  bf16 [B, H_kv, NC_cap, d]       updated in place, NC_cap >= ceil(T_cap / s)
 *   len_old, len_new, max_new_tokens         as sda_update_compressed_keys
 *   window   l, a multiple of stride, stride <= l <= 64
 *   stride   s in {8, 16, 32, 64}
 * Every entry whose window holds a token of [len_old[b], len_new[b]) is
 * recomputed from K (token-by-token updates equal a bulk build bit for bit).
 */
sda_status_t sda_update_compressed_keys_strided(const void* k, void* k_tilde,
                                                const int32_t* len_old, const int32_t* len_new,
                                                int max_new_tokens, int B, int H_kv, int d,
                                                int T_cap, int NC_cap, int window, int stride,
                                                void* stream);

/*
 * Indexer scoring on overlapping compressed keys, max-pooled onto the
 * 64-token block grid, then top-k and block-set assembly ([SparDA] eq. (6),
 * (9); §4.4 compression l = 32, s = 16; §4.3 and fig. 3: the compressed
 * scores are max-pooled to block scores):
 *   z_j = f . K~_j for every entry j < ceil(seq_len / s);
 *   S_J = max of z_j over the windows that share a token with block J
 *         (j*s < 64(J+1) and j*s + l > 64J);
 *   B = init U local U top_k(S over the other blocks) as in sda_score_select.
 *
 *   f          bf16 [B, NQ, H_kv, d]
 *   k_tilde    bf16 [B, H_kv, NC_cap, d] from sda_update_compressed_keys_strided
 *   window, stride  as that call
 *   scores_opt f32 [B, NQ, H_kv, NB_cap] out or NULL: pooled block scores, with
 *              NB_cap = ceil(NC_cap * stride / 64) (entries past nb undefined)
 *   other arguments as sda_score_select (1 <= seq_len <= stride * NC_cap).
 * Workspace: sda_score_select_pooled_workspace() bytes, with the same
 * zero-fill and no-overlap contract as sda_score_select.  With top_k <= 64
 * and NB_cap <= 4096 the selection runs inside the scoring launch, otherwise
 * as a second launch; the results are identical.
 */
size_t sda_score_select_pooled_workspace(int B, int NQ, int H_kv, int NC_cap, int stride, int top_k);
sda_status_t sda_score_select_pooled(const void* f, const void* k_tilde, const int32_t* seq_len,
                                     int B, int NQ, int H_kv, int d, int NC_cap, int window, int stride,
                                     int n_init, int n_local, int top_k, int n_sel_max,
                                     int32_t* block_idx, int32_t* n_sel, float* scores_opt,
                                     void* ws, size_t ws_bytes, void* stream);

/*
 * Block-sparse decode attention ([SparDA] eq. (7) and §4.2 step 4; [SSV] NSA
 * selection branch step 3): for every query head h of every row,
 *   O = softmax(q_h K_B^T * scale) V_B
 * over the tokens of the row's selected blocks that lie below seq_len[b].
 * Split-K over the block list with online softmax state (m, l, o) per split
 * and a log-sum-exp combine ([SSV] online-softmax section).
 *
 *   q          bf16 [B, NQ, H_q, d]
 *   k, v       bf16 [B, H_kv, T_cap, d]   (a cache, or a staging buffer with slot_opt)
 *   seq_len    i32  [B]
 *   block_idx  i32  [B, NQ, H_kv, n_sel_max] logical block ids (ascending not required)
 *   n_sel      i32  [B, NQ, H_kv]  entries used per row (<= n_sel_max)
 *   slot_opt   i32  [B, NQ, H_kv, n_sel_max] or NULL: the physical 64-token block of
 *              each entry inside the row's K/V buffer (NULL: the logical id itself)
 *   out        f32  [B, NQ, H_q, d];  lse_opt f32 [B, NQ, H_q] (natural log) or NULL
 *   split_k    splits per row (0 = chosen by the library)
 * Entries with ids outside [0, nb) or slots outside the buffer are skipped.
 * A row with no valid token gets out = 0 and lse = -inf.
 * Workspace: sda_sparse_decode_workspace() bytes (0 when one split per row).
 * It holds per-row arrival counters: zero-fill it before its first use; every
 * completed call leaves it zero-filled again.  Calls that share a workspace
 * must not overlap in time.
 */
size_t sda_sparse_decode_workspace(int B, int NQ, int H_q, int H_kv, int n_sel_max, int d, int split_k);
sda_status_t sda_sparse_decode(const void* q, const void* k, const void* v, const int32_t* seq_len,
                               const int32_t* block_idx, const int32_t* n_sel, int n_sel_max,
                               const int32_t* slot_opt, int T_cap,
                               int B, int NQ, int H_q, int H_kv, int d, float scale,
                               float* out, float* lse_opt, int split_k,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped verification decode ([SSV] core mechanism 1 and its verification
 * kernel algorithm): the NQ queries of a sequence form consecutive groups of
 * group_C (the last group may be smaller).  For each (batch, group, KV head)
 * the kernel loads each block of the group's merged set once and serves all
 * C*G query heads from it.
 *   SDA_GROUP_EXACT      merged set = union of the group's lists; query c
 *                        attends only to its own list (exact per-query result).
 *   SDA_GROUP_SHARED_REP every query attends to the group's first list.
 *   block_idx must be ascending per row (as sda_score_select writes it).
 *   union_count_opt i32 [B, ceil(NQ / group_C), H_kv] out or NULL: blocks loaded
 *   per group (size of the merged set, or of the first list in shared mode);
 *   written for group_C >= 2 only.
 * Other arguments (workspace contract included) as sda_sparse_decode.
 * Shared mode: group_C * G <= 32 and group_C <= 8.  Exact mode: group_C * G
 * up to 128 rows and group_C up to 32; groups of two or more queries run on
 * the row-tiled engine (the group's union walked once through LDS, shared
 * among split_k workgroups, 0 = chosen by the library), group_C = 1 is the
 * per-query decode.  NB_cap blocks of bitmap must fit in LDS beside two K/V
 * slots (NB_cap <= 16384 at d = 128), else SDA_ERR_UNSUPPORTED.
 */
size_t sda_grouped_decode_workspace(int B, int NQ, int H_q, int H_kv, int n_sel_max, int d, int NB_cap,
                                    int group_C, int mode, int split_k);
sda_status_t sda_grouped_decode(const void* q, const void* k, const void* v, const int32_t* seq_len,
                                const int32_t* block_idx, const int32_t* n_sel, int n_sel_max,
                                int T_cap, int NB_cap, int B, int NQ, int H_q, int H_kv, int d,
                                float scale, int group_C, int mode,
                                float* out, float* lse_opt, int32_t* union_count_opt,
                                int split_k, void* ws, size_t ws_bytes, void* stream);

/*
 * NSA verification output with its three branches in one launch ([SSV] NSA
 * three-branch derivation, steps 3-6; verification-kernel algorithm step 3c):
 * for every query head h of every query,
 *   o = g_c * Attn(q_h, K~, V~) + g_s * Attn(q_h, K_B, V_B) + g_w * Attn(q_h, K_win, V_win)
 * where the compressed branch attends to the ceil(seq_len / cmp_stride)
 * compressed keys and values present, the selection branch to the listed
 * blocks exactly as sda_grouped_decode (group_C, mode: the merged set loaded
 * once per group), and the window branch to tokens [seq_len - window, seq_len).
 * Each branch keeps its own softmax; the last workgroup of a row group merges
 * each branch's splits by log-sum-exp, normalises, and writes the gated sum.
 * With two or more queries per KV head, row tiles of as many whole groups as
 * fit in 128 rows and 32 queries (all NQ queries when they fit) load the
 * compressed cache and the window once per tile; the result is the same per
 * query as with tiles of one group.
 *
 *   q .. n_sel_max, T_cap   as sda_grouped_decode (NB_cap = ceil(T_cap / 64))
 *   group_C, mode  group_C <= 32 and group_C * G <= 128 (SDA_ERR_UNSUPPORTED
 *                  beyond)
 *   k_cmp, v_cmp  bf16 [B, H_kv, NC_cap, d]: compressed keys and values, e.g. from
 *                 sda_update_compressed_keys(_strided) applied to K and to V
 *   cmp_stride    tokens per compressed entry's stride (1..64), NC_cap >= ceil(T_cap / cmp_stride)
 *   window        w >= 0 tokens of the sliding-window branch (0: the branch is empty)
 *   gates         f32 [B, NQ, H_q, 3]: (g_c, g_s, g_w) per query head
 *   out           f32 [B, NQ, H_q, d]
 *   lse_opt       f32 [B, NQ, H_q, 3] or NULL: each branch's log-sum-exp (natural
 *                 log, -inf for a branch with no token; that branch contributes 0)
 *   union_count_opt  as sda_grouped_decode
 * Workspace: sda_nsa_decode_workspace() bytes (always > 0), with the
 * zero-fill and no-overlap contract of sda_sparse_decode.
 */
size_t sda_nsa_decode_workspace(int B, int NQ, int H_q, int H_kv, int n_sel_max, int d, int T_cap,
                                int NC_cap, int window, int group_C, int mode);
sda_status_t sda_nsa_decode(const void* q, const void* k, const void* v, const void* k_cmp, const void* v_cmp,
                            const int32_t* seq_len, const int32_t* block_idx, const int32_t* n_sel,
                            int n_sel_max, int T_cap, int NC_cap, int cmp_stride, int window,
                            const float* gates, int B, int NQ, int H_q, int H_kv, int d, float scale,
                            int group_C, int mode, float* out, float* lse_opt, int32_t* union_count_opt,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Refresh/reuse layer chain of NSA verification ([SSV] core mechanism 2 and
 * its scheduling algorithm): layers run in order on `stream`; a refresh
 * layer (refresh[j] != 0) routes first, s = f . K~ over its 64-token block
 * keys and top-n per row (sda_score_select with no initial or local blocks,
 * [SSV] NSA steps 1-2), and caches the lists in block_idx_cache /
 * n_sel_cache; every layer then runs sda_nsa_decode with the cached lists
 * (a reuse layer skips routing and inherits the latest refresh layer's
 * lists).  Refresh layers take two launches, reuse layers one.
 *
 *   layers   host array of L layer descriptors (below); k_route and f_route
 *            are read on refresh layers only
 *   refresh  host array of L flags; refresh[0] must be non-zero
 *   block_idx_cache i32 [B, NQ, H_kv, top_n], n_sel_cache i32 [B, NQ, H_kv]:
 *            the cache (left holding the last refresh layer's lists)
 *   other arguments as sda_nsa_decode (NB_cap = ceil(T_cap / 64) block keys
 *   per row in k_route)
 * Workspace: sda_nsa_chain_workspace() bytes, zero-filled before first use.
 */
typedef struct {
    const void* q;          /* bf16 [B, NQ, H_q, d] */
    const void* k;          /* bf16 [B, H_kv, T_cap, d] */
    const void* v;          /* bf16 [B, H_kv, T_cap, d] */
    const void* k_cmp;      /* bf16 [B, H_kv, NC_cap, d] compressed keys of the compressed branch */
    const void* v_cmp;      /* bf16 [B, H_kv, NC_cap, d] compressed values */
    const void* k_route;    /* bf16 [B, H_kv, NB_cap, d] block keys the router scores (refresh layers) */
    const void* f_route;    /* bf16 [B, NQ, H_kv, d] routing vectors (refresh layers) */
    const float* gates;     /* f32 [B, NQ, H_q, 3] */
    float* out;             /* f32 [B, NQ, H_q, d] */
    float* lse;             /* f32 [B, NQ, H_q, 3] or NULL */
} sda_nsa_layer;
size_t sda_nsa_chain_workspace(int B, int NQ, int H_q, int H_kv, int d, int T_cap, int NC_cap, int window,
                               int top_n, int group_C, int mode);
sda_status_t sda_nsa_chain(const sda_nsa_layer* layers, const uint8_t* refresh, int L, const int32_t* seq_len,
                           int B, int NQ, int H_q, int H_kv, int d, int T_cap, int NC_cap, int cmp_stride,
                           int window, int top_n, int group_C, int mode, float scale, int32_t* block_idx_cache,
                           int32_t* n_sel_cache, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step of the layer pipeline ([SparDA] §4.2 and eq. (6): layer l's
 * indexer vectors choose layer l+1's blocks while layer l attends).  The
 * block sets are those of sda_score_select(f_next, k_tilde_next, ...), bit for
 * bit; out and lse are those of sda_sparse_decode(q, k, v, ...) with one
 * query per sequence (NQ = 1) up to the order of summation (bit for bit when
 * both take the same launch shape, e.g. the same split_k).  One launch: the
 * workgroups of the decode come first; workgroups past them score layer
 * l+1's compressed keys (a 256-block chunk per four waves, at most two per
 * workgroup), keep each chunk's top-k and, in the last workgroup to finish a
 * row, merge the chunk lists into the row's block set.  When the lists do not
 * fit that (top_k > 64, NB_cap_next > 4096, or a launch shape of fewer than
 * four waves) it runs the two calls.
 *
 *   q .. split_k           as sda_sparse_decode (NQ = 1, no slot table)
 *   f_next .. n_sel_next   as sda_score_select for layer l+1 (NQ = 1);
 *                          block_idx_next / n_sel_next must not alias block_idx / n_sel
 *   k_tilde_cur            NULL, or layer l's compressed keys bf16 [B, H_kv, NB_cap_cur, d]:
 *                          the same launch refreshes the blocks touched by the tokens
 *                          [len_old_cur[b], seq_len[b]) from k, exactly as
 *                          sda_update_compressed_keys(k, k_tilde_cur, len_old_cur, seq_len,
 *                          max_new_tokens_cur, ...) does ([SparDA] §4.2 step 1: the key just
 *                          appended updates its block's mean); it must not alias k_tilde_next
 * Workspace: sda_decode_step_workspace() bytes, zero-filled before first use
 * (it holds arrival counters that every completed call leaves at zero).
 */
size_t sda_decode_step_workspace(int B, int H_q, int H_kv, int d, int n_sel_max, int split_k,
                                 int NB_cap_next, int top_k);
/* 1 if sda_decode_step with these sizes runs as one launch, 0 if it runs the
 * two calls (or the sizes are invalid). */
int sda_decode_step_is_fused(int B, int H_q, int H_kv, int d, int n_sel_max, int split_k,
                             int NB_cap_next, int top_k);
sda_status_t sda_decode_step(const void* q, const void* k, const void* v, const int32_t* seq_len,
                             const int32_t* block_idx, const int32_t* n_sel, int n_sel_max, int T_cap,
                             int B, int H_q, int H_kv, int d, float scale, float* out, float* lse_opt,
                             int split_k, const void* f_next, const void* k_tilde_next,
                             const int32_t* seq_len_next, int NB_cap_next, int n_init, int n_local, int top_k,
                             int n_sel_max_next, int32_t* block_idx_next, int32_t* n_sel_next,
                             void* k_tilde_cur, const int32_t* len_old_cur, int max_new_tokens_cur,
                             int NB_cap_cur, void* ws, size_t ws_bytes, void* stream);

/*
 * Prefill selection: a block set for every query position of a prefill
 * chunk ([SparDA] eq. (3): the set is a function of the query position, the
 * local window next to it; the complexity section's eq. (13) and (16) count
 * one selection over the compressed blocks per query token).  Query r sits
 * at position p = pos0 + r and chooses exactly as sda_score_select does for
 * a sequence of p + 1 tokens: blocks 0 .. p / 64 exist, {0..n_init-1} and
 * the last n_local of them are taken, and top-k ranks the others by
 * f_r . K~_j (fp32 sums of exact bf16 products; ties to the lower block id);
 * written ascending, padded with -1.  n_local >= 1 (the block holding the
 * query is always local), so every ranked block is complete at p and the
 * compressed keys of the whole sequence may be passed.
 *
 *   f          bf16 [B, NQ, H_kv, d]    one indexer vector per query position and KV head
 *   k_tilde    bf16 [B, H_kv, NB_cap, d] (64 * NB_cap >= pos0 + NQ)
 *   seq_len    i32  [B] cached tokens; a query at a position >= seq_len[b] gets no blocks
 *   pos0       position of query 0 (0 for a whole-sequence prefill; chunked
 *              prefill passes the chunk's start)
 *   block_idx  i32  [B, NQ, H_kv, n_sel_max] out; n_sel i32 [B, NQ, H_kv] out
 * Positions must stay below 32768 (a query's 512 block scores are kept in
 * registers); beyond that the call returns SDA_ERR_UNSUPPORTED.
 */
sda_status_t sda_prefill_select(const void* f, const void* k_tilde, const int32_t* seq_len, int B, int NQ, int H_kv,
                                int d, int NB_cap, int pos0, int n_init, int n_local, int top_k, int n_sel_max,
                                int32_t* block_idx, int32_t* n_sel, void* stream);

/*
 * Prefill attention: causal block-sparse attention for every query position
 * of a chunk ([SparDA] eq. (7) per query and the complexity section's eq.
 * (15): each query token attends to its own k blocks): query r at position
 * p = pos0 + r, head h, attends to the tokens of its listed blocks that lie
 * at or before p.  Tiles of min(32, 128 / G) consecutive positions share
 * one pass over the union of their lists, each block fetched once into LDS
 * for the tile and every row masked to its own list and its own position.
 *
 *   q          bf16 [B, NQ, H_q, d]
 *   k, v       bf16 [B, H_kv, T_cap, d] (pos0 + NQ <= T_cap)
 *   block_idx, n_sel  as sda_prefill_select writes them (ascending per row)
 *   out f32 [B, NQ, H_q, d]; lse_opt f32 [B, NQ, H_q] or NULL
 * A query with no visible token gets out = 0 and lse = -inf.
 * Workspace: none is needed (sda_prefill_attention_workspace() returns 0;
 * ws may be NULL and is not read).  Lists hold block ids below
 * ceil(T_cap / 64) <= NB_cap <= 16384.
 */
size_t sda_prefill_attention_workspace(int B, int NQ, int H_q, int H_kv, int n_sel_max, int d, int NB_cap);
sda_status_t sda_prefill_attention(const void* q, const void* k, const void* v, const int32_t* seq_len,
                                   const int32_t* block_idx, const int32_t* n_sel, int n_sel_max, int T_cap,
                                   int NB_cap, int B, int NQ, int H_q, int H_kv, int d, float scale, int pos0,
                                   float* out, float* lse_opt, void* ws, size_t ws_bytes, void* stream);

/*
 * sda_decode_step without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of sda_decode_step (same kernels, same launch plan, bit-identical
 * results).  The scratch the kernels need (split partials, arrival counters,
 * per-chunk candidate lists or scores) lives in a static device array of
 * SDA_NOALLOC_SCRATCH_BYTES per device (its first 64 KiB are arrival
 * counters), held until the process ends; a call whose scratch would not fit
 * returns SDA_ERR_WORKSPACE and launches nothing.  The call allocates nothing:
 * its first call on a device looks up the array's address and clears its
 * counter region with a fill kernel on `stream`.  Every call on a device
 * shares that device's array: calls that overlap in time on one GPU race
 * (order them on one stream).
 */
#define SDA_NOALLOC_SCRATCH_BYTES (8u << 20)
sda_status_t sda_decode_step_noalloc(const void* q, const void* k, const void* v, const int32_t* seq_len,
                                     const int32_t* block_idx, const int32_t* n_sel, int n_sel_max, int T_cap,
                                     int B, int H_q, int H_kv, int d, float scale, float* out, float* lse_opt,
                                     int split_k, const void* f_next, const void* k_tilde_next,
                                     const int32_t* seq_len_next, int NB_cap_next, int n_init, int n_local,
                                     int top_k, int n_sel_max_next, int32_t* block_idx_next, int32_t* n_sel_next,
                                     void* k_tilde_cur, const int32_t* len_old_cur, int max_new_tokens_cur,
                                     int NB_cap_cur, void* stream);

/*
 * Offloaded-KV decode chain with a persistent prefetch pool ([SparDA] §4.2,
 * the decode-step algorithm, steps 2-4 and 6; §4.5 and fig. 5; §4.6 for the
 * first layer).  The K/V of every layer stay in pinned host memory; the
 * compressed keys, queries and indexer vectors are on the GPU.  The call
 * starts a pool of `prefetch_workgroups` long-lived workgroups on
 * `side_stream` that wait for transfer requests, then runs the layers in
 * order on `stream`:
 *   layer 0 selects its own blocks with f_first (§4.6) and enqueues them;
 *   layer l scores layer l+1's compressed keys with its indexer vector f
 *     (lookahead), enqueues layer l+1's blocks (the pool copies them from host
 *     memory into one of two device stages while the stream goes on), waits
 *     for its own blocks' transfer, and attends over them from the stage.
 * Waits are bounded: a request that does not complete within about 3 s sets
 * an error word in the workspace (int at byte offset 8; 0 = no error) and the
 * chain finishes with undefined outputs for that layer.  On return `stream`
 * is ordered after the pool's exit (the caller may reuse the workspace).
 *
 *   layers    host array of L <= 32 layer descriptors (below)
 *   seq_len   i32 [B]; all layers hold seq_len[b] tokens
 *   n_init, n_local, top_k  the block budget of every layer
 *   f_first   bf16 [B, 1, H_kv, d]: layer 0's own indexer vectors
 *   prefetch_workgroups  the pool's size (the CU share of the transfer), 1..128: at
 *             most half of the compute units, so that the stream's launches
 *             always find units the spinning pool does not hold
 *   block_idx_opt  i32 [L, B, 1, H_kv, n_init + n_local + top_k] out or NULL:
 *             the block lists each layer attended
 * Workspace: sda_offload_chain_workspace() bytes (no zero-fill needed).
 */
typedef struct {
    const void* k_host;     /* bf16 [B, H_kv, T_cap, d], pinned host memory mapped for the device */
    const void* v_host;
    const void* k_tilde;    /* bf16 [B, H_kv, NB_cap, d] device: this layer's compressed keys */
    const void* q;          /* bf16 [B, 1, H_q, d] device */
    const void* f;          /* bf16 [B, 1, H_kv, d] device: this layer's indexer vectors (score layer l+1) */
    float* out;             /* f32 [B, 1, H_q, d] device */
    float* lse;             /* f32 [B, 1, H_q] device or NULL */
} sda_offload_layer;
size_t sda_offload_chain_workspace(int L, int B, int H_q, int H_kv, int d, int T_cap, int n_init, int n_local,
                                   int top_k);
sda_status_t sda_offload_chain(const sda_offload_layer* layers, int L, const int32_t* seq_len, int B, int H_q,
                               int H_kv, int d, int T_cap, int n_init, int n_local, int top_k, float scale,
                               const void* f_first, int prefetch_workgroups, int32_t* block_idx_opt, void* ws,
                               size_t ws_bytes, void* stream, void* side_stream);

/*
 * Offloaded-KV gather ([SparDA] §4.2 steps 3 and 6, §4.5): copy the K and V
 * rows of each row's selected blocks from pinned host memory into a compact
 * device staging buffer, with GPU loads over the host link, on the caller's
 * (side) stream; sda_sparse_decode then reads the stage through slot_out.
 *
 *   k_src, v_src  host bf16 [B, H_kv, T_cap, d]; must be pinned host memory
 *                 mapped for the device (hipHostMalloc / torch pin_memory)
 *   block_idx     i32 [B, H_kv, n_sel_max] (one query per sequence); n_sel i32 [B, H_kv]
 *   k_stage, v_stage  bf16 [B, H_kv, n_sel_max * 64, d] out
 *   slot_out      i32 [B, H_kv, n_sel_max] out: entry e lives in stage block e (-1 past n_sel)
 *   max_workgroups  upper bound on workgroups the copy occupies (0 = library choice)
 */
sda_status_t sda_gather_blocks(const void* k_src, const void* v_src,
                               const int32_t* block_idx, const int32_t* n_sel, int n_sel_max,
                               int B, int H_kv, int d, int T_cap,
                               void* k_stage, void* v_stage, int32_t* slot_out,
                               int max_workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDA_H */
