// C-ABI layer of libsda: argument validation, workspace sizing, launch
// selection.  Validation runs on the host before any HIP call, so every
// invalid-argument path returns without touching the GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <climits>
#include <initializer_list>
#include <string>

#include "../../include/sda.h"
#include "sda_internal.h"

using namespace sda;

namespace {

thread_local std::string g_err;

sda_status_t fail(sda_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sda_status_t fail(sda_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

sda_status_t hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return SDA_OK;
    return fail(SDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int kBlock = SDA_BLOCK_TOKENS;
constexpr int kMaxGridYZ = 65535;
constexpr int kMaxNBCap = 16384;      // select keeps <= 64 keys per lane
constexpr int kMaxSplits = 1024;
constexpr int kMaxListLen = 65536;   // entries per block list (4M tokens of selected context)
constexpr size_t kLdsBytes = 160 * 1024;

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// every count the kernels and the planners form in int (rows, row groups,
// blocks of all rows) must fit in int: the product of the given sizes, each
// at least 1, is checked before any of them is multiplied in int
bool fits_int(std::initializer_list<long long> xs) {
    long long p = 1;
    for (const long long x : xs) {
        if (x < 1 || p > INT_MAX / x) return false;
        p *= x;
    }
    return true;
}

// the sizes every attention-family workspace query and call share: row
// counts that fit in int, a supported head dim and GQA ratio, lists of at
// most kMaxListLen entries, split_k in [0, kMaxSplits]
bool attn_sizes_ok(int B, int NQ, int H_q, int H_kv, int n_sel_max, int d, int split_k) {
    return fits_int({B, NQ, H_q}) && H_kv >= 1 && H_q % H_kv == 0 && H_q / H_kv <= 32 && (d == 64 || d == 128) &&
           n_sel_max >= 1 && n_sel_max <= kMaxListLen && split_k >= 0 && split_k <= kMaxSplits;
}

#define REQUIRE(cond, st, ...)                    \
    do {                                          \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

sda_status_t check_d(int d) {
    REQUIRE(d == 64 || d == 128, SDA_ERR_UNSUPPORTED, "head dim d=%d: only 64 and 128 are supported", d);
    return SDA_OK;
}

sda_status_t check_heads(int H_q, int H_kv) {
    REQUIRE(H_q >= 1 && H_kv >= 1, SDA_ERR_SHAPE, "H_q=%d H_kv=%d must be >= 1", H_q, H_kv);
    REQUIRE(H_q % H_kv == 0, SDA_ERR_SHAPE, "H_q=%d is not a multiple of H_kv=%d", H_q, H_kv);
    REQUIRE(H_q / H_kv <= 32, SDA_ERR_UNSUPPORTED, "G=%d query heads per KV head: at most 32", H_q / H_kv);
    return SDA_OK;
}

// list length the grouped kernel plans for: the whole first list in shared
// mode; in exact mode the merged size at half overlap between neighbours,
// n (1 + (C-1)/2), a middle estimate (the real union is only known on the GPU)
int grouped_list_estimate(int C, int mode, int n_sel_max) {
    if (C <= 1 || mode == SDA_GROUP_SHARED_REP) return n_sel_max;
    return n_sel_max + (C - 1) * n_sel_max / 2;
}

// workspace of the split decode: [counters, 256-byte padded][(m, l) partials][o partials]
void set_workspace(AttnArgs& a, void* ws, size_t need, int tasks, int ns, int rp) {
    if (need == 0) {
        a.counters = nullptr;
        a.part_ml = a.part_o = nullptr;
        return;
    }
    char* base = static_cast<char*>(ws);
    const size_t cbytes = ((size_t)tasks * sizeof(int) + 255) / 256 * 256;
    a.counters = reinterpret_cast<int*>(base);
    a.part_ml = reinterpret_cast<float*>(base + cbytes);
    a.part_o = a.part_ml + (size_t)tasks * ns * rp * 2;
}

#define TRY(expr)                          \
    do {                                   \
        sda_status_t _st = (expr);         \
        if (_st != SDA_OK) return _st;     \
    } while (0)

}  // namespace

extern "C" {

const char* sda_status_string(sda_status_t s) {
    // a C caller may pass any int: read the bits, not an out-of-range enum value
    int v;
    memcpy(&v, &s, sizeof v);
    switch (v) {
        case SDA_OK: return "SDA_OK";
        case SDA_ERR_NULL: return "SDA_ERR_NULL";
        case SDA_ERR_SHAPE: return "SDA_ERR_SHAPE";
        case SDA_ERR_UNSUPPORTED: return "SDA_ERR_UNSUPPORTED";
        case SDA_ERR_WORKSPACE: return "SDA_ERR_WORKSPACE";
        case SDA_ERR_ALIGN: return "SDA_ERR_ALIGN";
        case SDA_ERR_HIP: return "SDA_ERR_HIP";
    }
    return "SDA_ERR_UNKNOWN";
}

const char* sda_last_error(void) { return g_err.c_str(); }

const char* sda_version(void) { return "sda 0.1 gfx950"; }

// ---------------------------------------------------------------------------
sda_status_t sda_update_compressed_keys(const void* k, void* k_tilde, const int32_t* len_old,
                                        const int32_t* len_new, int max_new_tokens, int B,
                                        int H_kv, int d, int T_cap, int NB_cap, void* stream) {
    REQUIRE(k && k_tilde && len_old && len_new, SDA_ERR_NULL, "update_compressed_keys: null pointer");
    TRY(check_d(d));
    REQUIRE(B >= 1 && H_kv >= 1 && T_cap >= 1, SDA_ERR_SHAPE, "B=%d H_kv=%d T_cap=%d must be >= 1", B, H_kv, T_cap);
    REQUIRE(NB_cap >= ceil_div(T_cap, kBlock), SDA_ERR_SHAPE, "NB_cap=%d < ceil(T_cap/64)=%d", NB_cap, ceil_div(T_cap, kBlock));
    REQUIRE((long long)B * H_kv <= kMaxGridYZ, SDA_ERR_SHAPE, "B*H_kv=%lld exceeds %d", (long long)B * H_kv, kMaxGridYZ);
    REQUIRE(max_new_tokens >= 0, SDA_ERR_SHAPE, "max_new_tokens=%d < 0", max_new_tokens);
    REQUIRE(aligned16(k) && aligned16(k_tilde), SDA_ERR_ALIGN, "k and k_tilde must be 16-byte aligned");
    REQUIRE(aligned4(len_old) && aligned4(len_new), SDA_ERR_ALIGN, "length arrays must be 4-byte aligned");
    if (max_new_tokens == 0) return SDA_OK;
    int blocks = ceil_div(max_new_tokens, kBlock) + 1;
    if (blocks > NB_cap) blocks = NB_cap;
    return hip_status(launch_update_compressed_keys(static_cast<const uint16_t*>(k), static_cast<uint16_t*>(k_tilde),
                                                    len_old, len_new,
                                                    blocks, B, H_kv, d, T_cap, NB_cap, kBlock, kBlock,
                                                    static_cast<hipStream_t>(stream)),
                      "update_compressed_keys launch");
}

static bool stride_ok(int stride) { return stride == 8 || stride == 16 || stride == 32 || stride == 64; }

// overlapping compression: window (kernel) and stride in tokens
static sda_status_t check_pool(int window, int stride) {
    REQUIRE(stride == 8 || stride == 16 || stride == 32 || stride == 64, SDA_ERR_UNSUPPORTED,
            "stride=%d: supported strides are 8, 16, 32 and 64 tokens", stride);
    REQUIRE(window >= stride && window <= 64 && window % stride == 0, SDA_ERR_UNSUPPORTED,
            "window=%d: must be a multiple of the stride (%d) and at most 64 tokens", window, stride);
    return SDA_OK;
}

sda_status_t sda_update_compressed_keys_strided(const void* k, void* k_tilde, const int32_t* len_old,
                                                const int32_t* len_new, int max_new_tokens, int B, int H_kv,
                                                int d, int T_cap, int NC_cap, int window, int stride,
                                                void* stream) {
    REQUIRE(k && k_tilde && len_old && len_new, SDA_ERR_NULL, "update_compressed_keys_strided: null pointer");
    TRY(check_d(d));
    TRY(check_pool(window, stride));
    REQUIRE(B >= 1 && H_kv >= 1 && T_cap >= 1, SDA_ERR_SHAPE, "B=%d H_kv=%d T_cap=%d must be >= 1", B, H_kv, T_cap);
    REQUIRE(NC_cap >= ceil_div(T_cap, stride), SDA_ERR_SHAPE, "NC_cap=%d < ceil(T_cap/stride)=%d", NC_cap,
            ceil_div(T_cap, stride));
    REQUIRE((long long)B * H_kv <= kMaxGridYZ, SDA_ERR_SHAPE, "B*H_kv=%lld exceeds %d", (long long)B * H_kv, kMaxGridYZ);
    REQUIRE(max_new_tokens >= 0, SDA_ERR_SHAPE, "max_new_tokens=%d < 0", max_new_tokens);
    REQUIRE(aligned16(k) && aligned16(k_tilde), SDA_ERR_ALIGN, "k and k_tilde must be 16-byte aligned");
    REQUIRE(aligned4(len_old) && aligned4(len_new), SDA_ERR_ALIGN, "length arrays must be 4-byte aligned");
    if (max_new_tokens == 0) return SDA_OK;
    // tokens [lo, lo + m) touch at most ceil(m / stride) + window / stride entries
    long long entries = (long long)ceil_div(max_new_tokens, stride) + window / stride;
    if (entries > NC_cap) entries = NC_cap;
    return hip_status(launch_update_compressed_keys(static_cast<const uint16_t*>(k), static_cast<uint16_t*>(k_tilde),
                                                    len_old, len_new, (int)entries, B, H_kv, d, T_cap, NC_cap,
                                                    window, stride, static_cast<hipStream_t>(stream)),
                      "update_compressed_keys_strided launch");
}

// ---------------------------------------------------------------------------
// [scores: B*NQ*H_kv*NB_cap f32][candidate keys: B*NQ*H_kv*chunks*top_k u64]
// [arrival counters: B*H_kv*vector tiles i32], each region padded to 256 B
static size_t pad256(size_t n) { return (n + 255) & ~(size_t)255; }
static size_t score_region_bytes(int B, int NQ, int H_kv, int NB_cap) {
    return pad256((size_t)B * NQ * H_kv * NB_cap * sizeof(float));
}
static size_t cand_region_bytes(int B, int NQ, int H_kv, int NB_cap, int top_k) {
    if (!fused_select_ok(NB_cap, top_k)) return 0;
    return pad256((size_t)B * NQ * H_kv * score_chunks(NB_cap) * top_k * sizeof(uint64_t));
}

size_t sda_score_select_workspace(int B, int NQ, int H_kv, int NB_cap, int top_k) {
    if (!fits_int({B, NQ, H_kv}) || NB_cap < 1 || NB_cap > kMaxNBCap || top_k < 0) return 0;
    return score_region_bytes(B, NQ, H_kv, NB_cap) + cand_region_bytes(B, NQ, H_kv, NB_cap, top_k) +
           (size_t)B * H_kv * score_tiles(NQ, NB_cap, B * H_kv) * sizeof(int);
}

static sda_status_t check_select_common(const void* k_tilde, const int32_t* seq_len, int B, int NQ,
                                        int H_kv, int d, int NB_cap, int n_init, int n_local, int top_k,
                                        int n_sel_max, const int32_t* block_idx, const int32_t* n_sel) {
    REQUIRE(k_tilde && seq_len && block_idx && n_sel, SDA_ERR_NULL, "score_select: null pointer");
    TRY(check_d(d));
    REQUIRE(B >= 1 && NQ >= 1 && H_kv >= 1 && NB_cap >= 1, SDA_ERR_SHAPE,
            "B=%d NQ=%d H_kv=%d NB_cap=%d must be >= 1", B, NQ, H_kv, NB_cap);
    REQUIRE(NB_cap <= kMaxNBCap, SDA_ERR_UNSUPPORTED, "NB_cap=%d exceeds %d blocks", NB_cap, kMaxNBCap);
    REQUIRE(n_init >= 0 && n_local >= 0 && top_k >= 0, SDA_ERR_SHAPE,
            "n_init=%d n_local=%d top_k=%d must be >= 0", n_init, n_local, top_k);
    REQUIRE(n_sel_max >= 1 && (long long)n_sel_max >= (long long)n_init + n_local + top_k, SDA_ERR_SHAPE,
            "n_sel_max=%d < n_init+n_local+top_k=%lld", n_sel_max, (long long)n_init + n_local + top_k);
    REQUIRE((long long)B * H_kv <= kMaxGridYZ, SDA_ERR_SHAPE, "B*H_kv exceeds %d", kMaxGridYZ);
    REQUIRE(fits_int({B, NQ, H_kv}), SDA_ERR_SHAPE, "B*NQ*H_kv exceeds the int range");
    REQUIRE(aligned16(k_tilde), SDA_ERR_ALIGN, "k_tilde must be 16-byte aligned");
    REQUIRE(aligned4(seq_len) && aligned4(block_idx) && aligned4(n_sel), SDA_ERR_ALIGN,
            "int32 arrays must be 4-byte aligned");
    return SDA_OK;
}

sda_status_t sda_score_select(const void* f, const void* k_tilde, const int32_t* seq_len, int B, int NQ,
                              int H_kv, int d, int NB_cap, int n_init, int n_local, int top_k,
                              int n_sel_max, int32_t* block_idx, int32_t* n_sel, float* scores_opt,
                              void* ws, size_t ws_bytes, void* stream) {
    REQUIRE(f, SDA_ERR_NULL, "score_select: f is null");
    TRY(check_select_common(k_tilde, seq_len, B, NQ, H_kv, d, NB_cap, n_init, n_local, top_k, n_sel_max,
                            block_idx, n_sel));
    REQUIRE(aligned16(f), SDA_ERR_ALIGN, "f must be 16-byte aligned");
    REQUIRE(ceil_div(NQ, 16) <= kMaxGridYZ, SDA_ERR_SHAPE, "NQ too large");
    const size_t need = sda_score_select_workspace(B, NQ, H_kv, NB_cap, top_k);
    REQUIRE(ws && ws_bytes >= need, SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0, need);
    REQUIRE(aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    REQUIRE(!scores_opt || aligned4(scores_opt), SDA_ERR_ALIGN, "scores_opt must be 4-byte aligned");
    char* base = static_cast<char*>(ws);
    float* scores_ws = reinterpret_cast<float*>(base);
    const size_t cand_off = score_region_bytes(B, NQ, H_kv, NB_cap);
    uint64_t* cand = reinterpret_cast<uint64_t*>(base + cand_off);
    int* counters = reinterpret_cast<int*>(base + cand_off + cand_region_bytes(B, NQ, H_kv, NB_cap, top_k));
    // one launch (the last scoring workgroup of each row merges per-chunk
    // candidate lists) unless the lists would be too long for it
    if (!fused_select_ok(NB_cap, top_k)) cand = nullptr, counters = nullptr;
    SelectArgs a{seq_len, nullptr, B * NQ * H_kv, NQ, H_kv, NB_cap, n_init, n_local, top_k, n_sel_max,
                 block_idx, n_sel};
    return hip_status(launch_score_select(static_cast<const uint16_t*>(f), static_cast<const uint16_t*>(k_tilde), a, B, d, scores_opt, scores_ws,
                                          cand, counters, static_cast<hipStream_t>(stream)),
                      "score/select launch");
}

// overlapping compression: [block scores f32, B*NQ*H_kv*NB_cap][candidate keys
// u64 (in-launch selection only)][arrival counters i32, B*H_kv*NQ], with
// NB_cap = ceil(NC_cap * stride / 64) blocks per row
static int pooled_nb_cap(int NC_cap, int stride) { return ceil_div((long long)NC_cap * stride, kBlock); }

size_t sda_score_select_pooled_workspace(int B, int NQ, int H_kv, int NC_cap, int stride, int top_k) {
    if (!fits_int({B, NQ, H_kv}) || !stride_ok(stride) || NC_cap < 1 || pooled_nb_cap(NC_cap, stride) > kMaxNBCap ||
        top_k < 0)
        return 0;
    const int NB_cap = pooled_nb_cap(NC_cap, stride);
    return score_region_bytes(B, NQ, H_kv, NB_cap) + cand_region_bytes(B, NQ, H_kv, NB_cap, top_k) +
           (size_t)B * H_kv * NQ * sizeof(int);
}

sda_status_t sda_score_select_pooled(const void* f, const void* k_tilde, const int32_t* seq_len, int B, int NQ,
                                     int H_kv, int d, int NC_cap, int window, int stride, int n_init, int n_local,
                                     int top_k, int n_sel_max, int32_t* block_idx, int32_t* n_sel,
                                     float* scores_opt, void* ws, size_t ws_bytes, void* stream) {
    REQUIRE(f, SDA_ERR_NULL, "score_select_pooled: f is null");
    TRY(check_pool(window, stride));
    REQUIRE(NC_cap >= 1 && NC_cap <= (1 << 24), SDA_ERR_SHAPE, "NC_cap=%d out of range", NC_cap);
    const int NB_cap = pooled_nb_cap(NC_cap, stride);
    TRY(check_select_common(k_tilde, seq_len, B, NQ, H_kv, d, NB_cap, n_init, n_local, top_k, n_sel_max,
                            block_idx, n_sel));
    REQUIRE(aligned16(f), SDA_ERR_ALIGN, "f must be 16-byte aligned");
    REQUIRE(NQ <= kMaxGridYZ, SDA_ERR_SHAPE, "NQ=%d exceeds %d", NQ, kMaxGridYZ);
    const size_t need = sda_score_select_pooled_workspace(B, NQ, H_kv, NC_cap, stride, top_k);
    REQUIRE(ws && ws_bytes >= need, SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0, need);
    REQUIRE(aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    REQUIRE(!scores_opt || aligned4(scores_opt), SDA_ERR_ALIGN, "scores_opt must be 4-byte aligned");
    char* base = static_cast<char*>(ws);
    float* scores_ws = reinterpret_cast<float*>(base);
    const size_t cand_off = score_region_bytes(B, NQ, H_kv, NB_cap);
    uint64_t* cand = reinterpret_cast<uint64_t*>(base + cand_off);
    int* counters = reinterpret_cast<int*>(base + cand_off + cand_region_bytes(B, NQ, H_kv, NB_cap, top_k));
    if (!fused_select_ok(NB_cap, top_k)) cand = nullptr, counters = nullptr;
    SelectArgs a{seq_len, nullptr, B * NQ * H_kv, NQ, H_kv, NB_cap, n_init, n_local, top_k, n_sel_max,
                 block_idx, n_sel};
    return hip_status(launch_score_select_pooled(static_cast<const uint16_t*>(f), static_cast<const uint16_t*>(k_tilde),
                                                 a, B, d, window, stride, NC_cap, scores_opt, scores_ws, cand,
                                                 counters, static_cast<hipStream_t>(stream)),
                      "pooled score/select launch");
}

// [z f32 and per-chunk statistics][scores f32, B*NQ*H_kv*NB_cap][candidate keys u64
// (in-launch selection only)][arrival counters i32, B*H_kv*NQ], 256-B aligned regions
size_t sda_score_select_multihead_workspace(int B, int NQ, int H_q, int H_kv, int NB_cap, int top_k) {
    if (!fits_int({B, NQ, H_q}) || H_kv < 1 || H_q % H_kv || NB_cap < 1 || NB_cap > kMaxNBCap || top_k < 0) return 0;
    return pad256(multihead_ws_floats(B, NQ, H_q, H_kv, NB_cap) * sizeof(float)) +
           score_region_bytes(B, NQ, H_kv, NB_cap) + cand_region_bytes(B, NQ, H_kv, NB_cap, top_k) +
           (size_t)B * H_kv * NQ * sizeof(int);
}

sda_status_t sda_score_select_multihead(const void* q, const void* k_tilde, const int32_t* seq_len, int B,
                                        int NQ, int H_q, int H_kv, int d, int NB_cap, int n_init, int n_local,
                                        int top_k, int n_sel_max, float tau, int32_t* block_idx,
                                        int32_t* n_sel, float* scores_opt, void* ws, size_t ws_bytes,
                                        void* stream) {
    REQUIRE(q, SDA_ERR_NULL, "score_select_multihead: q is null");
    TRY(check_select_common(k_tilde, seq_len, B, NQ, H_kv, d, NB_cap, n_init, n_local, top_k, n_sel_max,
                            block_idx, n_sel));
    TRY(check_heads(H_q, H_kv));
    REQUIRE(H_q / H_kv <= 16, SDA_ERR_UNSUPPORTED, "comparator supports G <= 16");
    REQUIRE(tau > 0.f && isfinite(tau), SDA_ERR_SHAPE, "tau must be finite and > 0");
    REQUIRE(aligned16(q), SDA_ERR_ALIGN, "q must be 16-byte aligned");
    REQUIRE((long long)NQ <= kMaxGridYZ, SDA_ERR_SHAPE, "NQ too large");
    const size_t need = sda_score_select_multihead_workspace(B, NQ, H_q, H_kv, NB_cap, top_k);
    REQUIRE(ws && ws_bytes >= need, SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0, need);
    REQUIRE(aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    REQUIRE(!scores_opt || aligned4(scores_opt), SDA_ERR_ALIGN, "scores_opt must be 4-byte aligned");
    char* base = static_cast<char*>(ws);
    float* z = reinterpret_cast<float*>(base);
    float* stats = reinterpret_cast<float*>(base + pad256((size_t)B * NQ * H_q * NB_cap * sizeof(float)));
    size_t off = pad256(multihead_ws_floats(B, NQ, H_q, H_kv, NB_cap) * sizeof(float));
    float* scores_ws = reinterpret_cast<float*>(base + off);
    off += score_region_bytes(B, NQ, H_kv, NB_cap);
    uint64_t* cand = reinterpret_cast<uint64_t*>(base + off);
    int* counters = reinterpret_cast<int*>(base + off + cand_region_bytes(B, NQ, H_kv, NB_cap, top_k));
    if (!fused_select_ok(NB_cap, top_k)) cand = nullptr, counters = nullptr;
    SelectArgs a{seq_len, nullptr, B * NQ * H_kv, NQ, H_kv, NB_cap, n_init, n_local, top_k, n_sel_max,
                 block_idx, n_sel};
    return hip_status(launch_multihead_select(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_tilde),
                                              a, B, H_q, d, tau, z, stats, scores_opt, scores_ws, cand, counters,
                                              static_cast<hipStream_t>(stream)),
                      "multihead score/select launch");
}

// InfLLM-V2's selector on overlapping compressed keys: [z and chunk statistics
// over the NC_cap entries][block scores][candidate keys][arrival counters]
size_t sda_score_select_multihead_pooled_workspace(int B, int NQ, int H_q, int H_kv, int NC_cap, int stride,
                                                   int top_k) {
    if (!fits_int({B, NQ, H_q}) || H_kv < 1 || H_q % H_kv || !stride_ok(stride) || NC_cap < 1 ||
        NC_cap > kMaxNBCap * (kBlock / stride) || top_k < 0)
        return 0;
    const int NB_cap = pooled_nb_cap(NC_cap, stride);
    return pad256(multihead_ws_floats(B, NQ, H_q, H_kv, NC_cap) * sizeof(float)) +
           score_region_bytes(B, NQ, H_kv, NB_cap) + cand_region_bytes(B, NQ, H_kv, NB_cap, top_k) +
           (size_t)B * H_kv * NQ * sizeof(int);
}

sda_status_t sda_score_select_multihead_pooled(const void* q, const void* k_tilde, const int32_t* seq_len, int B,
                                               int NQ, int H_q, int H_kv, int d, int NC_cap, int window, int stride,
                                               int n_init, int n_local, int top_k, int n_sel_max, float tau,
                                               int32_t* block_idx, int32_t* n_sel, float* scores_opt, void* ws,
                                               size_t ws_bytes, void* stream) {
    REQUIRE(q, SDA_ERR_NULL, "score_select_multihead_pooled: q is null");
    TRY(check_pool(window, stride));
    REQUIRE(NC_cap >= 1 && NC_cap <= (1 << 24), SDA_ERR_SHAPE, "NC_cap=%d out of range", NC_cap);
    const int NB_cap = pooled_nb_cap(NC_cap, stride);
    TRY(check_select_common(k_tilde, seq_len, B, NQ, H_kv, d, NB_cap, n_init, n_local, top_k, n_sel_max, block_idx,
                            n_sel));
    TRY(check_heads(H_q, H_kv));
    REQUIRE(H_q / H_kv <= 16, SDA_ERR_UNSUPPORTED, "comparator supports G <= 16");
    REQUIRE(tau > 0.f && isfinite(tau), SDA_ERR_SHAPE, "tau must be finite and > 0");
    REQUIRE(aligned16(q), SDA_ERR_ALIGN, "q must be 16-byte aligned");
    REQUIRE((long long)NQ <= kMaxGridYZ, SDA_ERR_SHAPE, "NQ too large");
    const size_t need = sda_score_select_multihead_pooled_workspace(B, NQ, H_q, H_kv, NC_cap, stride, top_k);
    REQUIRE(ws && ws_bytes >= need, SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0, need);
    REQUIRE(aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    REQUIRE(!scores_opt || aligned4(scores_opt), SDA_ERR_ALIGN, "scores_opt must be 4-byte aligned");
    char* base = static_cast<char*>(ws);
    float* z = reinterpret_cast<float*>(base);
    float* stats = reinterpret_cast<float*>(base + pad256((size_t)B * NQ * H_q * NC_cap * sizeof(float)));
    size_t off = pad256(multihead_ws_floats(B, NQ, H_q, H_kv, NC_cap) * sizeof(float));
    float* scores_ws = reinterpret_cast<float*>(base + off);
    off += score_region_bytes(B, NQ, H_kv, NB_cap);
    uint64_t* cand = reinterpret_cast<uint64_t*>(base + off);
    int* counters = reinterpret_cast<int*>(base + off + cand_region_bytes(B, NQ, H_kv, NB_cap, top_k));
    if (!fused_select_ok(NB_cap, top_k)) cand = nullptr, counters = nullptr;
    SelectArgs a{seq_len, nullptr, B * NQ * H_kv, NQ, H_kv, NB_cap, n_init, n_local, top_k, n_sel_max,
                 block_idx, n_sel};
    return hip_status(launch_multihead_select_pooled(static_cast<const uint16_t*>(q),
                                                     static_cast<const uint16_t*>(k_tilde), a, B, H_q, d, tau, window,
                                                     stride, NC_cap, z, stats, scores_opt, scores_ws, cand, counters,
                                                     static_cast<hipStream_t>(stream)),
                      "multihead pooled score/select launch");
}

// ---------------------------------------------------------------------------
size_t sda_sparse_decode_workspace(int B, int NQ, int H_q, int H_kv, int n_sel_max, int d, int split_k) {
    if (!attn_sizes_ok(B, NQ, H_q, H_kv, n_sel_max, d, split_k)) return 0;
    const int G = H_q / H_kv;
    const int rp = attn_rows_pad(1, G);
    const int tasks = B * NQ * H_kv;
    const AttnPlan p = attn_plan(d, rp, tasks, n_sel_max, 1, SDA_GROUP_EXACT, 1, n_sel_max, split_k);
    return attn_ws_bytes(tasks, p.n_split, rp, d);
}

static sda_status_t check_attn_common(const void* q, const void* k, const void* v, const int32_t* seq_len,
                                      const int32_t* block_idx, const int32_t* n_sel, int n_sel_max, int T_cap,
                                      int B, int NQ, int H_q, int H_kv, int d, float scale, float* out,
                                      int split_k) {
    REQUIRE(q && k && v && seq_len && block_idx && n_sel && out, SDA_ERR_NULL, "decode: null pointer");
    TRY(check_d(d));
    TRY(check_heads(H_q, H_kv));
    REQUIRE(B >= 1 && NQ >= 1 && T_cap >= 1 && n_sel_max >= 1, SDA_ERR_SHAPE,
            "B=%d NQ=%d T_cap=%d n_sel_max=%d must be >= 1", B, NQ, T_cap, n_sel_max);
    REQUIRE(n_sel_max <= kMaxListLen, SDA_ERR_UNSUPPORTED, "n_sel_max=%d exceeds %d entries", n_sel_max, kMaxListLen);
    REQUIRE(fits_int({B, NQ, H_q}), SDA_ERR_SHAPE, "B*NQ*H_q exceeds the int range");
    REQUIRE(split_k >= 0 && split_k <= kMaxSplits, SDA_ERR_SHAPE, "split_k=%d outside [0, %d]", split_k, kMaxSplits);
    REQUIRE(isfinite(scale) && scale > 0.f, SDA_ERR_SHAPE, "scale must be finite and > 0");
    REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), SDA_ERR_ALIGN,
            "q, k, v, out must be 16-byte aligned");
    REQUIRE(aligned4(seq_len) && aligned4(block_idx) && aligned4(n_sel), SDA_ERR_ALIGN,
            "int32 arrays must be 4-byte aligned");
    return SDA_OK;
}

sda_status_t sda_sparse_decode(const void* q, const void* k, const void* v, const int32_t* seq_len,
                               const int32_t* block_idx, const int32_t* n_sel, int n_sel_max,
                               const int32_t* slot_opt, int T_cap, int B, int NQ, int H_q, int H_kv, int d,
                               float scale, float* out, float* lse_opt, int split_k, void* ws, size_t ws_bytes,
                               void* stream) {
    TRY(check_attn_common(q, k, v, seq_len, block_idx, n_sel, n_sel_max, T_cap, B, NQ, H_q, H_kv, d, scale, out,
                          split_k));
    const long long tasks = (long long)B * NQ * H_kv;
    REQUIRE(tasks <= kMaxGridYZ, SDA_ERR_SHAPE, "B*NQ*H_kv=%lld exceeds %d", tasks, kMaxGridYZ);
    REQUIRE(!slot_opt || aligned4(slot_opt), SDA_ERR_ALIGN, "slot_opt must be 4-byte aligned");
    const int G = H_q / H_kv;
    const int rp = attn_rows_pad(1, G);
    const AttnPlan plan = attn_plan(d, rp, (int)tasks, n_sel_max, 1, SDA_GROUP_EXACT, 1, n_sel_max, split_k);
    const int ns = plan.n_split;
    const size_t need = attn_ws_bytes((int)tasks, ns, rp, d);
    REQUIRE(need == 0 || (ws && ws_bytes >= need), SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
            ws ? ws_bytes : 0, need);
    REQUIRE(need == 0 || aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    AttnArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.seq_len = seq_len;
    a.block_idx = block_idx;
    a.n_sel = n_sel;
    a.slot = slot_opt;
    a.out = out;
    a.lse = lse_opt;
    a.union_count = nullptr;
    set_workspace(a, ws, need, (int)tasks, ns, rp);
    a.n_sel_max = n_sel_max;
    a.T_cap = T_cap;
    a.NB_cap = ceil_div(T_cap, kBlock);
    a.B = B;
    a.NQ = NQ;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.G = G;
    a.d = d;
    a.C = 1;
    a.mode = SDA_GROUP_EXACT;
    a.n_groups = NQ;
    a.n_split = ns;
    a.waves = plan.waves;
    a.scale_log2 = scale * 1.4426950408889634f;
    return hip_status(launch_attention(a, static_cast<hipStream_t>(stream)), "sparse_decode launch");
}

// ---------------------------------------------------------------------------
// NSA three-branch verification output.  Launch shape: the most waves per
// workgroup that still let two workgroups share a compute unit (LDS of the V
// tiles and the merged lists, resident waves), and as many splits per row
// group as fill the two slots of every compute unit in one dispatch round
// (at least one per branch), shared among the branches in proportion to
// their blocks.  A branch's workgroup walks its blocks W apart, so the
// longest branch, not the launch as a whole, sets the pace; measured on the
// 64K verification workload this shape (4 waves, 2/1/1 splits) took 54 us
// against 62-92 us for shapes with a single slot per compute unit or one
// split for the 16-block compressed branch.
constexpr int kNsaMaxWaves = 10;                     // the attention kernel's waves per workgroup

// NSA verification of two or more queries per (batch, KV head) runs on the
// row-tiled engine (in shared mode every query takes its group's first
// list): a tile holds as many whole groups of group_C
// queries as fit in 128 rows and 32 queries (all of them when they fit), so
// the compressed cache and the window are loaded once per tile rather than
// once per group, and the listed blocks' union once per tile.  Every tile
// gets S >= 3 workgroups, which it shares among the branches at run time in
// proportion to their block counts; K/V slots as for grouped verification.
struct NsaTiles {
    int Cq, n_tiles, tiles, RW, S, nbuf;
};
// queries per verification tile: as many whole groups of group_C as fit in
// 128 rows (of G heads) and 32 queries, and no more than the groups of NQ
static int verify_tile_queries(int NQ, int group_C, int G) {
    return std::min((std::min(32, 128 / G) / group_C) * group_C, ceil_div(NQ, group_C) * group_C);
}
struct TilePlan {
    int S, nbuf;
};
static TilePlan grouped_tile_plan(int tiles, int d, int NB_cap, int split_k);
static NsaTiles nsa_tiles(int B, int NQ, int H_q, int H_kv, int d, int T_cap, int group_C, int mode) {
    NsaTiles t{};
    const int G = H_kv > 0 ? H_q / H_kv : 0;
    if (G < 1 || group_C < 1 || group_C > 32 || group_C * G > 128) return t;
    const int cq = verify_tile_queries(NQ, group_C, G);
    const int NB_cap = ceil_div(T_cap, kBlock);
    if (cq < 2 || tiled_grouped_bufs(d, NB_cap) < 2) return t;
    t.Cq = cq;
    t.n_tiles = ceil_div(NQ, cq);
    t.tiles = B * H_kv * t.n_tiles;
    t.RW = tiled_grouped_rw(cq * G);
    const TilePlan tp = grouped_tile_plan(t.tiles, d, NB_cap, 0);
    t.S = std::max(3, tp.S);
    t.nbuf = tp.nbuf;
    return t;
}
struct NsaPlan {
    AttnPlan p;
    int ns_c, ns_s, ns_w;
};
static NsaPlan nsa_plan(int d, int rp, int tasks, int group_C, int mode, int T_cap, int n_sel_max, int NC_cap,
                        int window) {
    NsaPlan n{};
    const int list = grouped_list_estimate(group_C, mode, n_sel_max);
    const int cmp_blocks = ceil_div(NC_cap, kBlock);
    const int win_blocks = window > 0 ? ceil_div(window, kBlock) + 1 : 0;    // a window may straddle one more block
    const int total = list + cmp_blocks + win_blocks;
    const int NB_cap = ceil_div(T_cap, kBlock);
    const int resident = rp == 16 ? 12 : 4;                 // waves per compute unit (VGPR-bound)
    int W = std::min(kNsaMaxWaves / 2, resident / 2);
    while (W > 1 && 2 * attn_smem_bytes_host(d, rp, W, group_C, mode, NB_cap, n_sel_max) > kLdsBytes) --W;
    const int S = std::max(3, (2 * kCUs) / std::max(tasks, 1));
    n.ns_c = std::min(cmp_blocks, std::max(1, (S * cmp_blocks + total / 2) / total));
    n.ns_w = std::max(1, std::min(win_blocks, (S * win_blocks + total / 2) / total));
    n.ns_s = std::min(std::max(list, 1), std::max(1, S - n.ns_c - n.ns_w));
    n.ns_c = std::max(1, n.ns_c);
    n.p = AttnPlan{W, n.ns_s};
    return n;
}

size_t sda_nsa_decode_workspace(int B, int NQ, int H_q, int H_kv, int n_sel_max, int d, int T_cap, int NC_cap,
                                int window, int group_C, int mode) {
    if (!attn_sizes_ok(B, NQ, H_q, H_kv, n_sel_max, d, 0) || group_C < 1 || group_C > 32 || T_cap < 1 ||
        ceil_div(T_cap, kBlock) > kMaxNBCap || NC_cap < 1 || window < 0 ||
        (mode != SDA_GROUP_EXACT && mode != SDA_GROUP_SHARED_REP))
        return 0;
    const NsaTiles nt = nsa_tiles(B, NQ, H_q, H_kv, d, T_cap, group_C, mode);
    if (nt.Cq) return tiled_ws_bytes(nt.tiles, nt.S, nt.RW, d);
    if (group_C > 8 || group_C * (H_q / H_kv) > 32) return 0;
    const int rp = attn_rows_pad(group_C, H_q / H_kv);
    const int tasks = B * ceil_div(NQ, group_C) * H_kv;
    const NsaPlan n = nsa_plan(d, rp, tasks, group_C, mode, T_cap, n_sel_max, NC_cap, window);
    return attn_ws_bytes(tasks, n.ns_c + n.ns_s + n.ns_w, rp, d);
}

sda_status_t sda_nsa_decode(const void* q, const void* k, const void* v, const void* k_cmp, const void* v_cmp,
                            const int32_t* seq_len, const int32_t* block_idx, const int32_t* n_sel, int n_sel_max,
                            int T_cap, int NC_cap, int cmp_stride, int window, const float* gates, int B, int NQ,
                            int H_q, int H_kv, int d, float scale, int group_C, int mode, float* out,
                            float* lse_opt, int32_t* union_count_opt, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_attn_common(q, k, v, seq_len, block_idx, n_sel, n_sel_max, T_cap, B, NQ, H_q, H_kv, d, scale, out,
                          0));
    REQUIRE(k_cmp && v_cmp && gates, SDA_ERR_NULL, "nsa_decode: compressed cache or gates is null");
    REQUIRE(aligned16(k_cmp) && aligned16(v_cmp), SDA_ERR_ALIGN, "k_cmp and v_cmp must be 16-byte aligned");
    REQUIRE(aligned4(gates) && (!lse_opt || aligned4(lse_opt)) && (!union_count_opt || aligned4(union_count_opt)),
            SDA_ERR_ALIGN, "gates, lse and union_count must be 4-byte aligned");
    REQUIRE(cmp_stride >= 1 && cmp_stride <= 64, SDA_ERR_UNSUPPORTED, "cmp_stride=%d outside [1, 64]", cmp_stride);
    REQUIRE(NC_cap >= ceil_div(T_cap, cmp_stride), SDA_ERR_SHAPE, "NC_cap=%d < ceil(T_cap/cmp_stride)=%d", NC_cap,
            ceil_div(T_cap, cmp_stride));
    REQUIRE(window >= 0, SDA_ERR_SHAPE, "window=%d < 0", window);
    REQUIRE(mode == SDA_GROUP_EXACT || mode == SDA_GROUP_SHARED_REP, SDA_ERR_SHAPE, "mode=%d", mode);
    REQUIRE(group_C >= 1 && group_C <= 32, SDA_ERR_UNSUPPORTED, "group_C=%d outside [1, 32]", group_C);
    REQUIRE(ceil_div(T_cap, kBlock) <= kMaxNBCap, SDA_ERR_UNSUPPORTED, "T_cap=%d beyond %d blocks", T_cap, kMaxNBCap);
    const int G = H_q / H_kv;
    const NsaTiles nt = nsa_tiles(B, NQ, H_q, H_kv, d, T_cap, group_C, mode);
    if (nt.Cq) {
        REQUIRE((long long)nt.tiles <= (1LL << 24), SDA_ERR_SHAPE, "B*tiles*H_kv=%d exceeds %d", nt.tiles, 1 << 24);
        const size_t need = tiled_ws_bytes(nt.tiles, nt.S, nt.RW, d);
        REQUIRE(ws && ws_bytes >= need, SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0,
                need);
        REQUIRE(aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
        TiledArgs t{};
        t.q = static_cast<const uint16_t*>(q);
        t.k = static_cast<const uint16_t*>(k);
        t.v = static_cast<const uint16_t*>(v);
        t.seq_len = seq_len;
        t.block_idx = block_idx;
        t.n_sel = n_sel;
        t.out = out;
        t.lse = lse_opt;
        t.n_sel_max = n_sel_max;
        t.T_cap = T_cap;
        t.NB_cap = ceil_div(T_cap, kBlock);
        t.B = B;
        t.NQ = NQ;
        t.H_q = H_q;
        t.H_kv = H_kv;
        t.G = G;
        t.Cq = nt.Cq;
        t.n_tiles = nt.n_tiles;
        t.bm_words = t.NB_cap;
        t.nbuf = nt.nbuf;
        t.scale_log2 = scale * 1.4426950408889634f;
        t.n_split = nt.S;
        t.union_count = union_count_opt;
        char* base = static_cast<char*>(ws);
        const size_t rows = (size_t)nt.tiles * nt.S * nt.RW * 16;
        t.counters = reinterpret_cast<int*>(base);
        t.part_ml = reinterpret_cast<float*>(base + pad256((size_t)nt.tiles * 4));
        t.part_o = t.part_ml + rows * 2;
        t.nsa = 1;
        t.kc = static_cast<const uint16_t*>(k_cmp);
        t.vc = static_cast<const uint16_t*>(v_cmp);
        t.gates = gates;
        t.NC_cap = NC_cap;
        t.cmp_stride = cmp_stride;
        t.window = window;
        t.Cu = group_C;
        t.n_ugroups = ceil_div(NQ, group_C);
        t.rep = mode == SDA_GROUP_SHARED_REP;
        return hip_status(launch_tiled_attention(t, d, static_cast<hipStream_t>(stream)), "nsa_decode launch");
    }
    REQUIRE(group_C * G <= 128, SDA_ERR_UNSUPPORTED, "group_C*G=%d exceeds 128 rows", group_C * G);
    REQUIRE(group_C <= 8 && group_C * G <= 32, SDA_ERR_UNSUPPORTED,
            "group_C=%d, G=%d: beyond 8 queries and 32 rows a group needs row tiles (two or more queries per "
            "KV head, a bitmap of %d blocks within LDS)", group_C, G, ceil_div(T_cap, kBlock));
    const int n_groups = ceil_div(NQ, group_C);
    const long long tasks = (long long)B * n_groups * H_kv;
    REQUIRE(tasks <= kMaxGridYZ, SDA_ERR_SHAPE, "B*groups*H_kv=%lld exceeds %d", tasks, kMaxGridYZ);
    const int rp = attn_rows_pad(group_C, G);
    const NsaPlan n = nsa_plan(d, rp, (int)tasks, group_C, mode, T_cap, n_sel_max, NC_cap, window);
    const int ns = n.ns_c + n.ns_s + n.ns_w;
    REQUIRE(ns <= kMaxSplits, SDA_ERR_UNSUPPORTED, "%d splits per row group exceed %d", ns, kMaxSplits);
    const size_t lds = attn_smem_bytes_host(d, rp, n.p.waves, group_C, mode, ceil_div(T_cap, kBlock), n_sel_max);
    REQUIRE(lds <= kLdsBytes, SDA_ERR_UNSUPPORTED, "group needs %zu bytes of LDS", lds);
    const size_t need = attn_ws_bytes((int)tasks, ns, rp, d);
    REQUIRE(ws && ws_bytes >= need, SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0, need);
    REQUIRE(aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    AttnArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.seq_len = seq_len;
    a.block_idx = block_idx;
    a.n_sel = n_sel;
    a.slot = nullptr;
    a.out = out;
    a.lse = lse_opt;
    a.union_count = union_count_opt;
    set_workspace(a, ws, need, (int)tasks, ns, rp);
    a.n_sel_max = n_sel_max;
    a.T_cap = T_cap;
    a.NB_cap = ceil_div(T_cap, kBlock);
    a.B = B;
    a.NQ = NQ;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.G = G;
    a.d = d;
    a.C = group_C;
    a.mode = mode;
    a.n_groups = n_groups;
    a.n_split = ns;
    a.waves = n.p.waves;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.nsa = 1;
    a.kc = static_cast<const uint16_t*>(k_cmp);
    a.vc = static_cast<const uint16_t*>(v_cmp);
    a.gates = gates;
    a.NC_cap = NC_cap;
    a.cmp_stride = cmp_stride;
    a.window = window;
    a.ns_c = n.ns_c;
    a.ns_s = n.ns_s;
    return hip_status(launch_attention(a, static_cast<hipStream_t>(stream)), "nsa_decode launch");
}

// ---------------------------------------------------------------------------
// decode step: layer l's decode and layer l+1's scoring and selection in one
// launch (workgroups past the attention grid score and select)
static bool step_fused_plan(int B, int H_q, int H_kv, int d, int n_sel_max, int split_k, int NB_cap_next,
                            int top_k, AttnPlan* plan) {
    if (!fused_select_ok(NB_cap_next, top_k)) return false;
    // the decode takes about half of the compute units, so that the scoring
    // workgroups run beside it from the start instead of after it (at 128K:
    // 2 splits, 28.5 us per step, against 30.7 us with the decode's own
    // choice of 4 splits over all units)
    const int tasks = B * H_kv;
    // (and at least four waves per workgroup: a scoring group needs them)
    const int sk = split_k > 0 ? split_k : max(1, min(kCUs / (2 * tasks), n_sel_max / 4));
    *plan = attn_plan(d, attn_rows_pad(1, H_q / H_kv), tasks, n_sel_max, 1, SDA_GROUP_EXACT, 1, n_sel_max, sk);
    // a scoring workgroup needs at least one group of four waves
    return plan->waves >= 4 &&
           step_lds_bytes(top_k, score_chunks(NB_cap_next), min(plan->waves / 4, 2)) <= 160 * 1024;
}

int sda_decode_step_is_fused(int B, int H_q, int H_kv, int d, int n_sel_max, int split_k, int NB_cap_next,
                             int top_k) {
    if (!attn_sizes_ok(B, 1, H_q, H_kv, n_sel_max, d, split_k) || NB_cap_next < 1 || NB_cap_next > kMaxNBCap ||
        top_k < 0)
        return 0;
    AttnPlan plan{};
    return step_fused_plan(B, H_q, H_kv, d, n_sel_max, split_k, NB_cap_next, top_k, &plan) ? 1 : 0;
}

size_t sda_decode_step_workspace(int B, int H_q, int H_kv, int d, int n_sel_max, int split_k, int NB_cap_next,
                                 int top_k) {
    if (!attn_sizes_ok(B, 1, H_q, H_kv, n_sel_max, d, split_k) || NB_cap_next < 1 || NB_cap_next > kMaxNBCap ||
        top_k < 0)
        return 0;
    AttnPlan plan{};
    size_t dec;
    if (step_fused_plan(B, H_q, H_kv, d, n_sel_max, split_k, NB_cap_next, top_k, &plan))
        dec = attn_ws_bytes(B * H_kv, plan.n_split, attn_rows_pad(1, H_q / H_kv), d);
    else
        dec = sda_sparse_decode_workspace(B, 1, H_q, H_kv, n_sel_max, d, split_k);
    return pad256(dec) + sda_score_select_workspace(B, 1, H_kv, NB_cap_next, top_k);
}

}  // extern "C"

namespace {

// The decode step's arguments, in the order of the C call.
struct StepCall {
    const void* q; const void* k; const void* v; const int32_t* seq_len;
    const int32_t* block_idx; const int32_t* n_sel; int n_sel_max; int T_cap;
    int B, H_q, H_kv, d; float scale; float* out; float* lse; int split_k;
    const void* f_next; const void* k_tilde_next; const int32_t* seq_len_next;
    int NB_cap_next, n_init, n_local, top_k, n_sel_max_next;
    int32_t* block_idx_next; int32_t* n_sel_next;
    void* k_tilde_cur; const int32_t* len_old_cur; int max_new_tokens_cur; int NB_cap_cur;
};

// Where the step's scratch lives: the decode's split partials and arrival
// counters, the scoring's scores, per-chunk candidate lists and arrival
// counters.  Counters must be zero before a call; every completed call
// leaves them zero.
struct StepScratch {
    int* dec_counters; float* part_ml; float* part_o;
    float* scores; uint64_t* cand; int* sel_counters;
};

// the decode's plan and partial-buffer bytes (counters excluded)
struct StepPlan {
    bool fused;
    AttnPlan plan;
    int tasks, rp;
    size_t partial_bytes;
};

StepPlan step_plan(const StepCall& c) {
    StepPlan sp{};
    sp.tasks = c.B * c.H_kv;
    sp.rp = attn_rows_pad(1, c.H_q / c.H_kv);
    sp.fused = step_fused_plan(c.B, c.H_q, c.H_kv, c.d, c.n_sel_max, c.split_k, c.NB_cap_next, c.top_k, &sp.plan);
    if (!sp.fused)
        sp.plan = attn_plan(c.d, sp.rp, sp.tasks, c.n_sel_max, 1, SDA_GROUP_EXACT, 1, c.n_sel_max, c.split_k);
    sp.partial_bytes = sp.plan.n_split > 1
                           ? (size_t)sp.tasks * sp.plan.n_split * sp.rp * ((size_t)c.d + 2) * sizeof(float)
                           : 0;
    return sp;
}

sda_status_t check_step(const StepCall& c) {
    TRY(check_attn_common(c.q, c.k, c.v, c.seq_len, c.block_idx, c.n_sel, c.n_sel_max, c.T_cap, c.B, 1, c.H_q,
                          c.H_kv, c.d, c.scale, c.out, c.split_k));
    REQUIRE(c.f_next, SDA_ERR_NULL, "decode_step: f_next is null");
    TRY(check_select_common(c.k_tilde_next, c.seq_len_next, c.B, 1, c.H_kv, c.d, c.NB_cap_next, c.n_init,
                            c.n_local, c.top_k, c.n_sel_max_next, c.block_idx_next, c.n_sel_next));
    REQUIRE(aligned16(c.f_next), SDA_ERR_ALIGN, "f_next must be 16-byte aligned");
    REQUIRE(c.block_idx_next != c.block_idx && c.n_sel_next != c.n_sel, SDA_ERR_SHAPE,
            "the next layer's block lists must not alias this layer's");
    REQUIRE((long long)c.B * c.H_kv <= kMaxGridYZ, SDA_ERR_SHAPE, "B*H_kv exceeds %d", kMaxGridYZ);
    if (c.k_tilde_cur) {                                   // this layer's compressed keys, refreshed in the launch
        REQUIRE(c.len_old_cur, SDA_ERR_NULL, "decode_step: len_old_cur is null");
        REQUIRE(c.k_tilde_cur != c.k_tilde_next, SDA_ERR_SHAPE, "this layer's compressed keys alias the next layer's");
        REQUIRE(c.NB_cap_cur >= ceil_div(c.T_cap, kBlock), SDA_ERR_SHAPE, "NB_cap_cur=%d < ceil(T_cap/64)=%d",
                c.NB_cap_cur, ceil_div(c.T_cap, kBlock));
        REQUIRE(c.max_new_tokens_cur >= 0, SDA_ERR_SHAPE, "max_new_tokens_cur=%d < 0", c.max_new_tokens_cur);
        REQUIRE(aligned16(c.k_tilde_cur) && aligned4(c.len_old_cur), SDA_ERR_ALIGN,
                "k_tilde_cur must be 16-byte and len_old_cur 4-byte aligned");
    }
    return SDA_OK;
}

// Runs a checked step with its scratch at `w`.
sda_status_t run_step(const StepCall& c, const StepPlan& sp, const StepScratch& w, hipStream_t s) {
    const bool refresh = c.k_tilde_cur && c.max_new_tokens_cur > 0;
    AttnArgs a{};
    a.q = static_cast<const uint16_t*>(c.q);
    a.k = static_cast<const uint16_t*>(c.k);
    a.v = static_cast<const uint16_t*>(c.v);
    a.seq_len = c.seq_len;
    a.block_idx = c.block_idx;
    a.n_sel = c.n_sel;
    a.slot = nullptr;
    a.out = c.out;
    a.lse = c.lse;
    a.union_count = nullptr;
    a.counters = sp.plan.n_split > 1 ? w.dec_counters : nullptr;
    a.part_ml = sp.plan.n_split > 1 ? w.part_ml : nullptr;
    a.part_o = sp.plan.n_split > 1 ? w.part_o : nullptr;
    a.n_sel_max = c.n_sel_max;
    a.T_cap = c.T_cap;
    a.NB_cap = ceil_div(c.T_cap, kBlock);
    a.B = c.B;
    a.NQ = 1;
    a.H_q = c.H_q;
    a.H_kv = c.H_kv;
    a.G = c.H_q / c.H_kv;
    a.d = c.d;
    a.C = 1;
    a.mode = SDA_GROUP_EXACT;
    a.n_groups = 1;
    a.n_split = sp.plan.n_split;
    a.waves = sp.plan.waves;
    a.scale_log2 = c.scale * 1.4426950408889634f;
    const SelectArgs sel{c.seq_len_next, nullptr, c.B * c.H_kv, 1, c.H_kv, c.NB_cap_next, c.n_init, c.n_local,
                         c.top_k, c.n_sel_max_next, c.block_idx_next, c.n_sel_next};
    if (!sp.fused) {                                     // the calls one after the other
        if (refresh) {
            int blocks = ceil_div(c.max_new_tokens_cur, kBlock) + 1;
            if (blocks > c.NB_cap_cur) blocks = c.NB_cap_cur;
            TRY(hip_status(launch_update_compressed_keys(static_cast<const uint16_t*>(c.k),
                                                         static_cast<uint16_t*>(c.k_tilde_cur), c.len_old_cur,
                                                         c.seq_len, blocks, c.B, c.H_kv, c.d, c.T_cap, c.NB_cap_cur,
                                                         kBlock, kBlock, s),
                           "decode_step: compressed-key refresh launch"));
        }
        TRY(hip_status(launch_score_select(static_cast<const uint16_t*>(c.f_next),
                                           static_cast<const uint16_t*>(c.k_tilde_next), sel, c.B, c.d, nullptr,
                                           w.scores, nullptr, nullptr, s),
                       "decode_step: score/select launch"));
        return hip_status(launch_attention(a, s), "decode_step: decode launch");
    }
    a.step.vec = static_cast<const uint16_t*>(c.f_next);
    a.step.kt = static_cast<const uint16_t*>(c.k_tilde_next);
    a.step.cand = w.cand;
    a.step.counters = w.sel_counters;
    a.step.sel = sel;
    a.step.cpr = score_chunks(c.NB_cap_next);
    a.step.per_wg = min(sp.plan.waves / 4, 2);
    // scoring workgroups take as many passes over their chunks (up to four)
    // as keep the launch to one dispatch round beside the decode's
    // workgroups: a second round of scoring workgroups waits for the first
    // to retire (at 128K: 2 passes, 24.9 against 25.8 us per step launch)
    {
        const int dec_wgs = c.B * c.H_kv * sp.plan.n_split;
        const int score_wgs = ceil_div((long long)c.B * c.H_kv * a.step.cpr, a.step.per_wg);
        const int room = std::max(1, kCUs - dec_wgs);
        a.step.passes = std::max(1, std::min(4, ceil_div(score_wgs, room)));
    }
    // m new tokens touch at most floor((m + 62) / 64) + 1 blocks (one for a single token)
    a.step.ref_kt = refresh ? static_cast<uint16_t*>(c.k_tilde_cur) : nullptr;
    a.step.ref_len_old = c.len_old_cur;
    a.step.ref_NB_cap = c.NB_cap_cur;
    a.step.ref_blocks = refresh ? std::min((c.max_new_tokens_cur + kBlock - 2) / kBlock + 1, c.NB_cap_cur) : 0;
    return hip_status(launch_attention(a, s), "decode_step launch");
}

}  // namespace

extern "C" {

sda_status_t sda_decode_step(const void* q, const void* k, const void* v, const int32_t* seq_len,
                             const int32_t* block_idx, const int32_t* n_sel, int n_sel_max, int T_cap, int B,
                             int H_q, int H_kv, int d, float scale, float* out, float* lse_opt, int split_k,
                             const void* f_next, const void* k_tilde_next, const int32_t* seq_len_next,
                             int NB_cap_next, int n_init, int n_local, int top_k, int n_sel_max_next,
                             int32_t* block_idx_next, int32_t* n_sel_next, void* k_tilde_cur,
                             const int32_t* len_old_cur, int max_new_tokens_cur, int NB_cap_cur, void* ws,
                             size_t ws_bytes, void* stream) {
    const StepCall c{q, k, v, seq_len, block_idx, n_sel, n_sel_max, T_cap, B, H_q, H_kv, d, scale, out, lse_opt,
                     split_k, f_next, k_tilde_next, seq_len_next, NB_cap_next, n_init, n_local, top_k,
                     n_sel_max_next, block_idx_next, n_sel_next, k_tilde_cur, len_old_cur, max_new_tokens_cur,
                     NB_cap_cur};
    TRY(check_step(c));
    const size_t need = sda_decode_step_workspace(B, H_q, H_kv, d, n_sel_max, split_k, NB_cap_next, top_k);
    REQUIRE(ws && ws_bytes >= need, SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0, need);
    REQUIRE(aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    const StepPlan sp = step_plan(c);
    // [decode: counters, (m, l), o][score_select's layout: scores, candidate lists, counters]
    const size_t dec = attn_ws_bytes(sp.tasks, sp.plan.n_split, sp.rp, d);
    AttnArgs dw{};
    set_workspace(dw, ws, dec, sp.tasks, sp.plan.n_split, sp.rp);
    char* sws = static_cast<char*>(ws) + pad256(dec);
    const size_t cand_off = score_region_bytes(B, 1, H_kv, NB_cap_next);
    StepScratch w{dw.counters, dw.part_ml, dw.part_o, reinterpret_cast<float*>(sws),
                  reinterpret_cast<uint64_t*>(sws + cand_off),
                  reinterpret_cast<int*>(sws + cand_off + cand_region_bytes(B, 1, H_kv, NB_cap_next, top_k))};
    return run_step(c, sp, w, static_cast<hipStream_t>(stream));
}

sda_status_t sda_decode_step_noalloc(const void* q, const void* k, const void* v, const int32_t* seq_len,
                                     const int32_t* block_idx, const int32_t* n_sel, int n_sel_max, int T_cap,
                                     int B, int H_q, int H_kv, int d, float scale, float* out, float* lse_opt,
                                     int split_k, const void* f_next, const void* k_tilde_next,
                                     const int32_t* seq_len_next, int NB_cap_next, int n_init, int n_local,
                                     int top_k, int n_sel_max_next, int32_t* block_idx_next, int32_t* n_sel_next,
                                     void* k_tilde_cur, const int32_t* len_old_cur, int max_new_tokens_cur,
                                     int NB_cap_cur, void* stream) {
    const StepCall c{q, k, v, seq_len, block_idx, n_sel, n_sel_max, T_cap, B, H_q, H_kv, d, scale, out, lse_opt,
                     split_k, f_next, k_tilde_next, seq_len_next, NB_cap_next, n_init, n_local, top_k,
                     n_sel_max_next, block_idx_next, n_sel_next, k_tilde_cur, len_old_cur, max_new_tokens_cur,
                     NB_cap_cur};
    TRY(check_step(c));
    const StepPlan sp = step_plan(c);
    // [counter region: decode counters | selection counters][split partials][candidate lists or scores]
    const size_t dec_cnt = pad256((size_t)sp.tasks * sizeof(int));
    const size_t sel_cnt = (size_t)B * H_kv * sizeof(int);
    const size_t cand = (size_t)B * H_kv * score_chunks(NB_cap_next) * top_k * sizeof(uint64_t);
    const size_t scores = (size_t)B * H_kv * NB_cap_next * sizeof(float);
    const size_t data = pad256(sp.partial_bytes) + pad256(sp.fused ? cand : scores);
    REQUIRE(dec_cnt + sel_cnt <= kNoallocCounterBytes && data <= kNoallocScratchBytes - kNoallocCounterBytes,
            SDA_ERR_WORKSPACE,
            "decode_step_noalloc: the call needs %zu bytes of counters and %zu of data; the static scratch holds "
            "%zu and %zu (use sda_decode_step with a workspace)",
            dec_cnt + sel_cnt, data, kNoallocCounterBytes, kNoallocScratchBytes - kNoallocCounterBytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = nullptr;
    TRY(hip_status(noalloc_scratch(s, &base), "decode_step_noalloc: scratch set-up"));
    char* dat = base + kNoallocCounterBytes;
    float* part_ml = reinterpret_cast<float*>(dat);
    float* part_o = part_ml + (size_t)sp.tasks * sp.plan.n_split * sp.rp * 2;
    char* sel = dat + pad256(sp.partial_bytes);
    StepScratch w{reinterpret_cast<int*>(base), part_ml, part_o, reinterpret_cast<float*>(sel),
                  reinterpret_cast<uint64_t*>(sel), reinterpret_cast<int*>(base + dec_cnt)};
    return run_step(c, sp, w, s);
}

// ---------------------------------------------------------------------------
// refresh/reuse NSA layer chain: [routing workspace | NSA workspace]
size_t sda_nsa_chain_workspace(int B, int NQ, int H_q, int H_kv, int d, int T_cap, int NC_cap, int window,
                               int top_n, int group_C, int mode) {
    if (T_cap < 1 || top_n < 1) return 0;
    const size_t nsa = sda_nsa_decode_workspace(B, NQ, H_q, H_kv, top_n, d, T_cap, NC_cap, window, group_C, mode);
    const size_t sel = sda_score_select_workspace(B, NQ, H_kv, ceil_div(T_cap, kBlock), top_n);
    if (nsa == 0 || sel == 0) return 0;
    return pad256(sel) + nsa;
}

sda_status_t sda_nsa_chain(const sda_nsa_layer* layers, const uint8_t* refresh, int L, const int32_t* seq_len,
                           int B, int NQ, int H_q, int H_kv, int d, int T_cap, int NC_cap, int cmp_stride,
                           int window, int top_n, int group_C, int mode, float scale, int32_t* block_idx_cache,
                           int32_t* n_sel_cache, void* ws, size_t ws_bytes, void* stream) {
    REQUIRE(layers && refresh && seq_len && block_idx_cache && n_sel_cache, SDA_ERR_NULL, "nsa_chain: null pointer");
    REQUIRE(L >= 1, SDA_ERR_SHAPE, "nsa_chain: L=%d < 1", L);
    REQUIRE(refresh[0] != 0, SDA_ERR_SHAPE, "nsa_chain: the first layer must refresh (nothing is cached yet)");
    REQUIRE(top_n >= 1, SDA_ERR_SHAPE, "nsa_chain: top_n=%d < 1", top_n);
    for (int j = 0; j < L; ++j) {
        const sda_nsa_layer& y = layers[j];
        REQUIRE(y.q && y.k && y.v && y.k_cmp && y.v_cmp && y.gates && y.out, SDA_ERR_NULL,
                "nsa_chain: layer %d has a null pointer", j);
        REQUIRE(!refresh[j] || (y.k_route && y.f_route), SDA_ERR_NULL,
                "nsa_chain: refresh layer %d needs k_route and f_route", j);
    }
    const size_t need = sda_nsa_chain_workspace(B, NQ, H_q, H_kv, d, T_cap, NC_cap, window, top_n, group_C, mode);
    REQUIRE(need > 0, SDA_ERR_SHAPE, "nsa_chain: invalid sizes");
    REQUIRE(ws && ws_bytes >= need, SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0, need);
    REQUIRE(aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    const int NB_cap = ceil_div(T_cap, kBlock);
    const size_t sel = pad256(sda_score_select_workspace(B, NQ, H_kv, NB_cap, top_n));
    char* base = static_cast<char*>(ws);
    for (int j = 0; j < L; ++j) {
        const sda_nsa_layer& y = layers[j];
        if (refresh[j])
            TRY(sda_score_select(y.f_route, y.k_route, seq_len, B, NQ, H_kv, d, NB_cap, 0, 0, top_n, top_n,
                                 block_idx_cache, n_sel_cache, nullptr, base, sel, stream));
        TRY(sda_nsa_decode(y.q, y.k, y.v, y.k_cmp, y.v_cmp, seq_len, block_idx_cache, n_sel_cache, top_n, T_cap,
                           NC_cap, cmp_stride, window, y.gates, B, NQ, H_q, H_kv, d, scale, group_C, mode, y.out, y.lse,
                           nullptr, base + sel, ws_bytes - sel, stream));
    }
    return SDA_OK;
}

// ---------------------------------------------------------------------------
// prefill: per-token selection and causal block-sparse attention
sda_status_t sda_prefill_select(const void* f, const void* k_tilde, const int32_t* seq_len, int B, int NQ, int H_kv,
                                int d, int NB_cap, int pos0, int n_init, int n_local, int top_k, int n_sel_max,
                                int32_t* block_idx, int32_t* n_sel, void* stream) {
    REQUIRE(f, SDA_ERR_NULL, "prefill_select: f is null");
    TRY(check_select_common(k_tilde, seq_len, B, NQ, H_kv, d, NB_cap, n_init, n_local, top_k, n_sel_max, block_idx,
                            n_sel));
    REQUIRE(aligned16(f), SDA_ERR_ALIGN, "f must be 16-byte aligned");
    REQUIRE(n_local >= 1, SDA_ERR_SHAPE, "prefill_select: n_local=%d; the block holding a query must be local (>= 1)",
            n_local);
    REQUIRE(pos0 >= 0, SDA_ERR_SHAPE, "pos0=%d < 0", pos0);
    REQUIRE((long long)pos0 + NQ <= (long long)kBlock * NB_cap, SDA_ERR_SHAPE,
            "positions up to %lld exceed the compressed-key capacity of %lld tokens", (long long)pos0 + NQ - 1,
            (long long)kBlock * NB_cap);
    REQUIRE((long long)pos0 + NQ <= (long long)kBlock * kPrefillMaxBlocks, SDA_ERR_UNSUPPORTED,
            "prefill_select keeps a query's block scores in registers: positions must stay below %d",
            kBlock * kPrefillMaxBlocks);
    const PrefillSelectArgs a{static_cast<const uint16_t*>(f), static_cast<const uint16_t*>(k_tilde), seq_len, B, NQ,
                              H_kv, NB_cap, pos0, n_init, n_local, top_k, n_sel_max, block_idx, n_sel};
    return hip_status(launch_prefill_select(a, d, static_cast<hipStream_t>(stream)), "prefill_select launch");
}

size_t sda_prefill_attention_workspace(int B, int NQ, int H_q, int H_kv, int n_sel_max, int d, int NB_cap) {
    // the row-tiled engine merges nothing across workgroups: no workspace
    (void)B, (void)NQ, (void)H_q, (void)H_kv, (void)n_sel_max, (void)d, (void)NB_cap;
    return 0;
}

sda_status_t sda_prefill_attention(const void* q, const void* k, const void* v, const int32_t* seq_len,
                                   const int32_t* block_idx, const int32_t* n_sel, int n_sel_max, int T_cap,
                                   int NB_cap, int B, int NQ, int H_q, int H_kv, int d, float scale, int pos0,
                                   float* out, float* lse_opt, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_attn_common(q, k, v, seq_len, block_idx, n_sel, n_sel_max, T_cap, B, NQ, H_q, H_kv, d, scale, out, 0));
    REQUIRE(pos0 >= 0 && (long long)pos0 + NQ <= T_cap, SDA_ERR_SHAPE,
            "query positions [%d, %lld) must lie inside the cache capacity T_cap=%d", pos0, (long long)pos0 + NQ, T_cap);
    REQUIRE(NB_cap >= ceil_div(T_cap, kBlock) && NB_cap <= kMaxNBCap, SDA_ERR_SHAPE,
            "NB_cap=%d must lie in [ceil(T_cap/64), %d]", NB_cap, kMaxNBCap);
    const int G = H_q / H_kv;
    // the row-tiled engine: up to 128 rows of consecutive positions per
    // workgroup, every block of their union fetched once into LDS
    const int bm_words = std::min(NB_cap, ceil_div((long long)pos0 + NQ, kBlock));
    REQUIRE(tiled_lds_bytes(d, bm_words, 2) <= kTiledLdsMax, SDA_ERR_UNSUPPORTED,
            "a block bitmap of %d words does not fit in LDS", bm_words);
    TiledArgs t{};
    t.q = static_cast<const uint16_t*>(q);
    t.k = static_cast<const uint16_t*>(k);
    t.v = static_cast<const uint16_t*>(v);
    t.seq_len = seq_len;
    t.block_idx = block_idx;
    t.n_sel = n_sel;
    t.out = out;
    t.lse = lse_opt;
    t.n_sel_max = n_sel_max;
    t.T_cap = T_cap;
    t.NB_cap = NB_cap;
    t.B = B;
    t.NQ = NQ;
    t.H_q = H_q;
    t.H_kv = H_kv;
    t.G = G;
    t.Cq = tiled_queries_per_tile(G);
    t.n_tiles = ceil_div(NQ, t.Cq);
    t.prefill = 1;
    t.pos0 = pos0;
    t.bm_words = bm_words;
    t.nbuf = 2;
    t.scale_log2 = scale * 1.4426950408889634f;
    t.n_split = 1;
    REQUIRE(fits_int({B, H_kv, t.n_tiles}), SDA_ERR_SHAPE, "too many query tiles");
    (void)ws;
    (void)ws_bytes;
    return hip_status(launch_tiled_attention(t, d, static_cast<hipStream_t>(stream)), "prefill_attention launch");
}

// Exact grouped verification of two or more queries (C * G up to 128 rows, C
// up to 32) runs on the row-tiled engine: the group's union walked once
// through LDS, shared among S workgroups (split-K) so that a few groups still
// fill the chip.
static bool grouped_on_tiles(int group_C, int G, int mode) {
    return mode == SDA_GROUP_EXACT && group_C >= 2 && group_C * G <= 128 && group_C <= 32;
}
// Splits and K/V slots: one workgroup per compute unit with as many slots as
// LDS holds (up to four), S = CUs / tiles; when that leaves fewer than four
// splits and two-slot workgroups fit twice per compute unit, two slots and
// twice the splits.
static TilePlan grouped_tile_plan(int tiles, int d, int NB_cap, int split_k) {
    const int nb_max = tiled_grouped_bufs(d, NB_cap);
    const bool two_fit = 2 * tiled_lds_bytes(d, NB_cap, 2) <= kTiledLdsMax;
    tiles = std::max(tiles, 1);
    if (split_k > 0) {
        const int S = std::min(split_k, 64);
        return TilePlan{S, ((long long)tiles * S > kCUs && two_fit) ? 2 : nb_max};
    }
    const int S1 = std::max(1, std::min(16, kCUs / tiles));
    if (S1 < 4 && two_fit) return TilePlan{std::max(1, std::min(16, 2 * kCUs / tiles)), 2};
    return TilePlan{S1, nb_max};
}

// queries per tile of exact grouped verification: as many whole groups as
// fit in 128 rows (of G heads) and 32 queries, as for NSA
static int grouped_tile_queries(int NQ, int group_C, int G) { return verify_tile_queries(NQ, group_C, G); }

size_t sda_grouped_decode_workspace(int B, int NQ, int H_q, int H_kv, int n_sel_max, int d, int NB_cap,
                                    int group_C, int mode, int split_k) {
    if (!attn_sizes_ok(B, NQ, H_q, H_kv, n_sel_max, d, split_k) || group_C < 1 || group_C > 32 || NB_cap < 1 ||
        NB_cap > kMaxNBCap || (mode != SDA_GROUP_EXACT && mode != SDA_GROUP_SHARED_REP))
        return 0;
    const int G = H_q / H_kv;
    const int n_groups = ceil_div(NQ, group_C);
    const int tasks = B * n_groups * H_kv;
    if (grouped_on_tiles(group_C, G, mode)) {
        const int cq = grouped_tile_queries(NQ, group_C, G);
        const int tiles = B * ceil_div(NQ, cq) * H_kv;
        return tiled_ws_bytes(tiles, grouped_tile_plan(tiles, d, NB_cap, split_k).S, tiled_grouped_rw(cq * G), d);
    }
    if (group_C > 8 || group_C * G > 32) return 0;
    const int rp = attn_rows_pad(group_C, G);
    const AttnPlan p = attn_plan(d, rp, tasks, grouped_list_estimate(group_C, mode, n_sel_max), group_C, mode,
                                 NB_cap, n_sel_max, split_k);
    return attn_ws_bytes(tasks, p.n_split, rp, d);
}

sda_status_t sda_grouped_decode(const void* q, const void* k, const void* v, const int32_t* seq_len,
                                const int32_t* block_idx, const int32_t* n_sel, int n_sel_max, int T_cap,
                                int NB_cap, int B, int NQ, int H_q, int H_kv, int d, float scale, int group_C,
                                int mode, float* out, float* lse_opt, int32_t* union_count_opt, int split_k,
                                void* ws, size_t ws_bytes, void* stream) {
    TRY(check_attn_common(q, k, v, seq_len, block_idx, n_sel, n_sel_max, T_cap, B, NQ, H_q, H_kv, d, scale, out,
                          split_k));
    REQUIRE(mode == SDA_GROUP_EXACT || mode == SDA_GROUP_SHARED_REP, SDA_ERR_SHAPE, "mode=%d", mode);
    const int G = H_q / H_kv;
    REQUIRE(NB_cap >= ceil_div(T_cap, kBlock) && NB_cap <= kMaxNBCap, SDA_ERR_SHAPE,
            "NB_cap=%d must lie in [ceil(T_cap/64), %d]", NB_cap, kMaxNBCap);
    REQUIRE(!union_count_opt || aligned4(union_count_opt), SDA_ERR_ALIGN, "union_count must be 4-byte aligned");
    REQUIRE(group_C >= 1 && group_C <= 32, SDA_ERR_UNSUPPORTED, "group_C=%d outside [1, 32]", group_C);
    const int n_groups = ceil_div(NQ, group_C);
    const long long tasks = (long long)B * n_groups * H_kv;
    if (grouped_on_tiles(group_C, G, mode)) {
        REQUIRE(tasks <= (1LL << 24), SDA_ERR_SHAPE, "B*groups*H_kv=%lld exceeds %d", tasks, 1 << 24);
        // tiles of several whole groups: the union of the tile's lists is
        // loaded once and every row masked to its own list, with the union
        // counted per group (groups of 4 at the 64K verification workload:
        // 25.8 against 27.1 us with a tile per group, alternated on one box)
        const int cq = grouped_tile_queries(NQ, group_C, G);
        const int n_tiles = ceil_div(NQ, cq);
        const int tiles = B * n_tiles * H_kv;
        const int RW = tiled_grouped_rw(cq * G);
        REQUIRE(tiled_grouped_bufs(d, NB_cap) >= 2, SDA_ERR_UNSUPPORTED, "NB_cap=%d: bitmap beyond LDS", NB_cap);
        const TilePlan tp = grouped_tile_plan(tiles, d, NB_cap, split_k);
        const int S = tp.S;
        const size_t need = tiled_ws_bytes(tiles, S, RW, d);
        REQUIRE(need == 0 || (ws && ws_bytes >= need), SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
                ws ? ws_bytes : 0, need);
        REQUIRE(need == 0 || aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
        TiledArgs t{};
        t.q = static_cast<const uint16_t*>(q);
        t.k = static_cast<const uint16_t*>(k);
        t.v = static_cast<const uint16_t*>(v);
        t.seq_len = seq_len;
        t.block_idx = block_idx;
        t.n_sel = n_sel;
        t.out = out;
        t.lse = lse_opt;
        t.n_sel_max = n_sel_max;
        t.T_cap = T_cap;
        t.NB_cap = NB_cap;
        t.B = B;
        t.NQ = NQ;
        t.H_q = H_q;
        t.H_kv = H_kv;
        t.G = G;
        t.Cq = cq;
        t.n_tiles = n_tiles;
        t.Cu = group_C;
        t.n_ugroups = n_groups;
        t.prefill = 0;
        t.pos0 = 0;
        t.bm_words = NB_cap;
        t.nbuf = tp.nbuf;
        t.scale_log2 = scale * 1.4426950408889634f;
        t.n_split = S;
        t.union_count = union_count_opt;
        if (need) {
            char* base = static_cast<char*>(ws);
            const size_t rows = (size_t)tiles * S * RW * 16;
            t.counters = reinterpret_cast<int*>(base);
            t.part_ml = reinterpret_cast<float*>(base + pad256((size_t)tiles * 4));
            t.part_o = t.part_ml + rows * 2;
        }
        return hip_status(launch_tiled_attention(t, d, static_cast<hipStream_t>(stream)), "grouped_decode launch");
    }
    REQUIRE(group_C <= 8, SDA_ERR_UNSUPPORTED, "group_C=%d outside [1, 8]", group_C);
    REQUIRE(group_C * G <= 32, SDA_ERR_UNSUPPORTED,
            "group_C*G=%d exceeds 32 rows (up to 128 are supported in exact mode)", group_C * G);
    REQUIRE(tasks <= kMaxGridYZ, SDA_ERR_SHAPE, "B*groups*H_kv=%lld exceeds %d", tasks, kMaxGridYZ);
    const int rp = attn_rows_pad(group_C, G);
    const AttnPlan plan = attn_plan(d, rp, (int)tasks, grouped_list_estimate(group_C, mode, n_sel_max), group_C,
                                    mode, NB_cap, n_sel_max, split_k);
    const size_t lds = attn_smem_bytes_host(d, rp, plan.waves, group_C, mode, NB_cap, n_sel_max);
    REQUIRE(lds <= kLdsBytes, SDA_ERR_UNSUPPORTED, "group needs %zu bytes of LDS", lds);
    const int ns = plan.n_split;
    const size_t need = attn_ws_bytes((int)tasks, ns, rp, d);
    REQUIRE(need == 0 || (ws && ws_bytes >= need), SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed",
            ws ? ws_bytes : 0, need);
    REQUIRE(need == 0 || aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    AttnArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.seq_len = seq_len;
    a.block_idx = block_idx;
    a.n_sel = n_sel;
    a.slot = nullptr;
    a.out = out;
    a.lse = lse_opt;
    a.union_count = union_count_opt;
    set_workspace(a, ws, need, (int)tasks, ns, rp);
    a.n_sel_max = n_sel_max;
    a.T_cap = T_cap;
    a.NB_cap = NB_cap;
    a.B = B;
    a.NQ = NQ;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.G = G;
    a.d = d;
    a.C = group_C;
    a.mode = mode;
    a.n_groups = n_groups;
    a.n_split = ns;
    a.waves = plan.waves;
    a.scale_log2 = scale * 1.4426950408889634f;
    return hip_status(launch_attention(a, static_cast<hipStream_t>(stream)), "grouped_decode launch");
}

// ---------------------------------------------------------------------------
// offloaded decode chain with the persistent prefetch pool.  Workspace:
// [control words, 256 B][lists: L x rows x nsm][n_sel: L x rows][slots: 2 x rows x nsm]
// [K stages: 2][V stages: 2][score_select workspace][decode workspace]
namespace {

struct ChainLayout {
    size_t ctrl, lists, nsel, slots, kst, vst, sel, dec, total;
    size_t stage_bytes, sel_bytes, dec_bytes;
};

ChainLayout chain_layout(int L, int B, int H_q, int H_kv, int d, int T_cap, int nsm, int top_k) {
    ChainLayout c{};
    const size_t rows = (size_t)B * H_kv;
    const int NB_cap = ceil_div(T_cap, kBlock);
    c.stage_bytes = pad256(rows * nsm * kBlock * d * 2);
    c.sel_bytes = pad256(sda_score_select_workspace(B, 1, H_kv, NB_cap, top_k));
    c.dec_bytes = pad256(sda_sparse_decode_workspace(B, 1, H_q, H_kv, nsm, d, 0));
    c.ctrl = 0;
    c.lists = 256;
    c.nsel = c.lists + pad256((size_t)L * rows * nsm * 4);
    c.slots = c.nsel + pad256((size_t)L * rows * 4);
    c.kst = c.slots + pad256(2 * rows * nsm * 4);
    c.vst = c.kst + 2 * c.stage_bytes;
    c.sel = c.vst + 2 * c.stage_bytes;
    c.dec = c.sel + c.sel_bytes;
    c.total = c.dec + c.dec_bytes;
    return c;
}

constexpr int kPfSpinLimit = 1 << 20;          // polls of ~3.4 us each before a wait gives up

}  // namespace

size_t sda_offload_chain_workspace(int L, int B, int H_q, int H_kv, int d, int T_cap, int n_init, int n_local,
                                   int top_k) {
    const long long nsm = (long long)n_init + n_local + top_k;
    if (L < 1 || L > kMaxChainLayers || !attn_sizes_ok(B, 1, H_q, H_kv, 1, d, 0) || T_cap < 1 ||
        ceil_div(T_cap, kBlock) > kMaxNBCap || n_init < 0 || n_local < 0 || top_k < 0 || nsm < 1 || nsm > kMaxListLen)
        return 0;
    return chain_layout(L, B, H_q, H_kv, d, T_cap, n_init + n_local + top_k, top_k).total;
}

sda_status_t sda_offload_chain(const sda_offload_layer* layers, int L, const int32_t* seq_len, int B, int H_q,
                               int H_kv, int d, int T_cap, int n_init, int n_local, int top_k, float scale,
                               const void* f_first, int prefetch_workgroups, int32_t* block_idx_opt, void* ws,
                               size_t ws_bytes, void* stream, void* side_stream) {
    REQUIRE(layers && seq_len && f_first, SDA_ERR_NULL, "offload_chain: null pointer");
    REQUIRE(L >= 1 && L <= kMaxChainLayers, SDA_ERR_SHAPE, "offload_chain: L=%d outside [1, %d]", L, kMaxChainLayers);
    // at most half of the compute units: the stream's own launches must always
    // find units that no pool workgroup occupies
    REQUIRE(prefetch_workgroups >= 1 && prefetch_workgroups <= kCUs / 2, SDA_ERR_SHAPE,
            "prefetch_workgroups=%d outside [1, %d]", prefetch_workgroups, kCUs / 2);
    REQUIRE(side_stream != stream, SDA_ERR_SHAPE, "offload_chain: the pool needs a stream of its own");
    TRY(check_d(d));
    TRY(check_heads(H_q, H_kv));
    REQUIRE(B >= 1 && T_cap >= 1 && n_init >= 0 && n_local >= 0 && top_k >= 0, SDA_ERR_SHAPE,
            "offload_chain: bad sizes");
    REQUIRE((long long)n_init + n_local + top_k >= 1 && (long long)n_init + n_local + top_k <= kMaxListLen,
            SDA_ERR_SHAPE, "offload_chain: n_init+n_local+top_k outside [1, %d]", kMaxListLen);
    const int nsm = n_init + n_local + top_k;
    const int NB_cap = ceil_div(T_cap, kBlock);
    REQUIRE((long long)B * H_kv <= kMaxGridYZ, SDA_ERR_SHAPE, "B*H_kv exceeds %d", kMaxGridYZ);
    REQUIRE(aligned16(f_first), SDA_ERR_ALIGN, "f_first must be 16-byte aligned");
    const ChainLayout c = chain_layout(L, B, H_q, H_kv, d, T_cap, nsm, top_k);
    REQUIRE(ws && ws_bytes >= c.total, SDA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : 0,
            c.total);
    REQUIRE(aligned16(ws), SDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    PrefetchArgs pa{};
    char* base = static_cast<char*>(ws);
    int* ctrl = reinterpret_cast<int*>(base + c.ctrl);
    const int rows = B * H_kv;
    int32_t* lists = block_idx_opt ? block_idx_opt : reinterpret_cast<int32_t*>(base + c.lists);
    int32_t* nsel = reinterpret_cast<int32_t*>(base + c.nsel);
    for (int j = 0; j < L; ++j) {
        const sda_offload_layer& y = layers[j];
        REQUIRE(y.k_host && y.v_host && y.k_tilde && y.q && y.f && y.out, SDA_ERR_NULL,
                "offload_chain: layer %d has a null pointer", j);
        REQUIRE(aligned16(y.k_tilde) && aligned16(y.q) && aligned16(y.f) && aligned16(y.out) &&
                    aligned16(y.k_host) && aligned16(y.v_host),
                SDA_ERR_ALIGN, "offload_chain: layer %d buffers must be 16-byte aligned", j);
        void* kd = nullptr;
        void* vd = nullptr;
        hipError_t e = hipHostGetDevicePointer(&kd, const_cast<void*>(y.k_host), 0);
        if (e == hipSuccess) e = hipHostGetDevicePointer(&vd, const_cast<void*>(y.v_host), 0);
        if (e != hipSuccess)
            return fail(SDA_ERR_HIP, "offload_chain: layer %d K/V are not pinned, device-mapped host memory: %s", j,
                        hipGetErrorString(e));
        PrefetchLayer& p = pa.layer[j];
        p.k_src = static_cast<const uint16_t*>(kd);
        p.v_src = static_cast<const uint16_t*>(vd);
        p.block_idx = lists + (size_t)j * rows * nsm;
        p.n_sel = nsel + (size_t)j * rows;
        p.k_stage = reinterpret_cast<uint16_t*>(base + c.kst + (j & 1) * c.stage_bytes);
        p.v_stage = reinterpret_cast<uint16_t*>(base + c.vst + (j & 1) * c.stage_bytes);
        p.slot = reinterpret_cast<int32_t*>(base + c.slots) + (size_t)(j & 1) * rows * nsm;
    }
    pa.L = L;
    pa.rows = rows;
    pa.n_sel_max = nsm;
    pa.T_cap = T_cap;
    pa.ctrl = ctrl;
    pa.spin_limit = kPfSpinLimit;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipStream_t side = static_cast<hipStream_t>(side_stream);
    char* sws = base + c.sel;
    // the score_select workspace holds arrival counters: clear them (and the
    // control words) on the stream before anything uses them
    TRY(hip_status(launch_prefetch_reset(ctrl, s), "offload_chain: reset"));
    TRY(hip_status(launch_zero_words(sws, c.sel_bytes + c.dec_bytes, s), "offload_chain: workspace clear"));
    // the pool starts after the reset, on its own stream
    hipEvent_t ev_start = nullptr, ev_end = nullptr;
    TRY(hip_status(hipEventCreateWithFlags(&ev_start, hipEventDisableTiming), "offload_chain: event"));
    hipError_t e = hipEventCreateWithFlags(&ev_end, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ev_start, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, ev_start, 0);
    if (e == hipSuccess) e = launch_prefetch_pool(pa, d, prefetch_workgroups, side);
    if (e == hipSuccess) e = hipEventRecord(ev_end, side);
    if (e != hipSuccess) {
        (void)hipEventDestroy(ev_start);
        if (ev_end) (void)hipEventDestroy(ev_end);
        return hip_status(e, "offload_chain: pool launch");
    }
    sda_status_t st = SDA_OK;
    const int total = rows * nsm;
    const size_t stage_tokens = (size_t)nsm * kBlock;
    auto run = [&]() -> sda_status_t {
        // layer 0 selects its own blocks with f_first
        TRY(sda_score_select(f_first, layers[0].k_tilde, seq_len, B, 1, H_kv, d, NB_cap, n_init, n_local, top_k, nsm,
                             lists, nsel, nullptr, sws, c.sel_bytes, stream));
        TRY(hip_status(launch_prefetch_enqueue(ctrl, 0, s), "offload_chain: enqueue"));
        for (int l = 0; l < L; ++l) {
            if (l + 1 < L) {                               // lookahead: layer l's vectors pick layer l+1's blocks
                TRY(sda_score_select(layers[l].f, layers[l + 1].k_tilde, seq_len, B, 1, H_kv, d, NB_cap, n_init,
                                     n_local, top_k, nsm, lists + (size_t)(l + 1) * rows * nsm,
                                     nsel + (size_t)(l + 1) * rows, nullptr, sws, c.sel_bytes, stream));
                TRY(hip_status(launch_prefetch_enqueue(ctrl, l + 1, s), "offload_chain: enqueue"));
            }
            TRY(hip_status(launch_prefetch_wait(ctrl, l, total, kPfSpinLimit, s), "offload_chain: wait"));
            const PrefetchLayer& p = pa.layer[l];
            TRY(sda_sparse_decode(layers[l].q, p.k_stage, p.v_stage, seq_len, p.block_idx, p.n_sel, nsm, p.slot,
                                  (int)stage_tokens, B, 1, H_q, H_kv, d, scale, layers[l].out, layers[l].lse, 0,
                                  c.dec_bytes ? base + c.dec : nullptr, c.dec_bytes, stream));
        }
        return SDA_OK;
    };
    st = run();
    // end the pool (also after an error) and order the stream after its exit
    e = launch_prefetch_stop(ctrl, s);
    hipError_t e2 = hipStreamWaitEvent(s, ev_end, 0);
    (void)hipEventDestroy(ev_start);
    (void)hipEventDestroy(ev_end);
    if (st != SDA_OK) return st;
    if (e == hipSuccess) e = e2;
    return hip_status(e, "offload_chain: pool stop");
}

// ---------------------------------------------------------------------------
sda_status_t sda_gather_blocks(const void* k_src, const void* v_src, const int32_t* block_idx,
                               const int32_t* n_sel, int n_sel_max, int B, int H_kv, int d, int T_cap,
                               void* k_stage, void* v_stage, int32_t* slot_out, int max_workgroups,
                               void* stream) {
    REQUIRE(k_src && v_src && block_idx && n_sel && k_stage && v_stage && slot_out, SDA_ERR_NULL,
            "gather_blocks: null pointer");
    TRY(check_d(d));
    REQUIRE(B >= 1 && H_kv >= 1 && n_sel_max >= 1 && T_cap >= 1, SDA_ERR_SHAPE,
            "B=%d H_kv=%d n_sel_max=%d T_cap=%d must be >= 1", B, H_kv, n_sel_max, T_cap);
    REQUIRE(max_workgroups >= 0, SDA_ERR_SHAPE, "max_workgroups=%d < 0", max_workgroups);
    REQUIRE(fits_int({B, H_kv, n_sel_max}), SDA_ERR_SHAPE, "B*H_kv*n_sel_max exceeds the int range");
    REQUIRE(aligned16(k_src) && aligned16(v_src) && aligned16(k_stage) && aligned16(v_stage), SDA_ERR_ALIGN,
            "source and stage buffers must be 16-byte aligned");
    REQUIRE(aligned4(block_idx) && aligned4(n_sel) && aligned4(slot_out), SDA_ERR_ALIGN,
            "int32 arrays must be 4-byte aligned");
    void* kd = nullptr;
    void* vd = nullptr;
    hipError_t e = hipHostGetDevicePointer(&kd, const_cast<void*>(k_src), 0);
    if (e != hipSuccess)
        return fail(SDA_ERR_HIP, "k_src is not pinned, device-mapped host memory: %s", hipGetErrorString(e));
    e = hipHostGetDevicePointer(&vd, const_cast<void*>(v_src), 0);
    if (e != hipSuccess)
        return fail(SDA_ERR_HIP, "v_src is not pinned, device-mapped host memory: %s", hipGetErrorString(e));
    return hip_status(launch_gather(static_cast<const uint16_t*>(kd), static_cast<const uint16_t*>(vd), block_idx,
                                    n_sel, n_sel_max, B, H_kv, d, T_cap, static_cast<uint16_t*>(k_stage),
                                    static_cast<uint16_t*>(v_stage), slot_out, max_workgroups,
                                    static_cast<hipStream_t>(stream)),
                      "gather launch");
}

}  // extern "C"
