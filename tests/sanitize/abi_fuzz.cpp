// Host-side fuzz of the C ABI's argument validation, built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code only (the device code is
// built as usual and never runs: the program refuses to start where a GPU is
// visible).  Every entry point of sda.h is called many times with arguments
// drawn from edge values (null and misaligned pointers, zero, negative, huge
// and overflowing sizes, non-finite floats); each call must return a status
// in the enum's range with a readable error string, and the sanitizers abort
// on any out-of-bounds access, integer overflow or other undefined behaviour
// in the validation and sizing code.  Without a device, a call whose
// arguments pass validation ends at its first HIP call with SDA_ERR_HIP.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>

#include "sda.h"

namespace {

std::mt19937_64 rng(20260624);
alignas(256) unsigned char arena[1 << 20];
constexpr int kLayers = 32;
sda_nsa_layer nsa_layers[kLayers];
sda_offload_layer off_layers[kLayers];
uint8_t refresh_flags[kLayers];
long long calls = 0, errors_seen[8] = {0};

int pick(int n) { return (int)(rng() % (unsigned)n); }

bool plausible = false;     // draw sizes that often pass validation (reach the deeper checks)

void* any_ptr() {
    if (plausible) return arena + 256 * pick(2048);
    switch (pick(16)) {
        case 0: return nullptr;
        case 1: return arena + 2 + 16 * pick(1024);            // misaligned
        default: return arena + 256 * pick(2048);
    }
}

template <class T> T draw();
template <> int draw<int>() {
    if (plausible && pick(8)) {
        static const int ok[] = {0, 1, 2, 3, 4, 8, 16, 32, 64, 128, 1024, 4096, 65536};
        return ok[pick(sizeof(ok) / sizeof(ok[0]))];
    }
    static const int edge[] = {-1, 0, 1, 2, 3, 4, 7, 8, 16, 31, 32, 33, 64, 65, 100, 128, 256, 4096, 4097,
                               32768, 65535, 65536, 1 << 20, 1 << 24, std::numeric_limits<int>::max(),
                               std::numeric_limits<int>::min()};
    return pick(4) == 0 ? (int)(rng() % 200) - 20 : edge[pick(sizeof(edge) / sizeof(edge[0]))];
}
template <> size_t draw<size_t>() {
    if (plausible && pick(4)) return std::numeric_limits<size_t>::max();
    static const size_t edge[] = {0, 1, 16, 256, 4096, 1u << 20, (size_t)1 << 40, std::numeric_limits<size_t>::max()};
    return edge[pick(sizeof(edge) / sizeof(edge[0]))];
}
template <> float draw<float>() {
    if (plausible && pick(4)) return 0.088388f;
    static const float edge[] = {0.f, 1.f, -1.f, 0.088388f, 11.3f, INFINITY, -INFINITY, NAN, 1e-30f};
    return edge[pick(sizeof(edge) / sizeof(edge[0]))];
}
template <> sda_status_t draw<sda_status_t>() { return (sda_status_t)(pick(10) - 2); }
template <> const void* draw<const void*>() { return any_ptr(); }
template <> void* draw<void*>() { return any_ptr(); }
template <> const int32_t* draw<const int32_t*>() { return static_cast<const int32_t*>(any_ptr()); }
template <> int32_t* draw<int32_t*>() { return static_cast<int32_t*>(any_ptr()); }
template <> const float* draw<const float*>() { return static_cast<const float*>(any_ptr()); }
template <> float* draw<float*>() { return static_cast<float*>(any_ptr()); }
template <> const uint8_t* draw<const uint8_t*>() { return pick(16) ? refresh_flags : nullptr; }
template <> const sda_nsa_layer* draw<const sda_nsa_layer*>() { return pick(16) ? nsa_layers : nullptr; }
template <> const sda_offload_layer* draw<const sda_offload_layer*>() { return pick(16) ? off_layers : nullptr; }

void reshuffle_layers() {
    for (int j = 0; j < kLayers; ++j) {
        nsa_layers[j] = sda_nsa_layer{any_ptr(), any_ptr(), any_ptr(), any_ptr(), any_ptr(),
                                      any_ptr(), any_ptr(), static_cast<const float*>(any_ptr()),
                                      static_cast<float*>(any_ptr()), static_cast<float*>(any_ptr())};
        off_layers[j] = sda_offload_layer{any_ptr(), any_ptr(), any_ptr(), any_ptr(), any_ptr(),
                                          static_cast<float*>(any_ptr()), static_cast<float*>(any_ptr())};
        refresh_flags[j] = (uint8_t)pick(2);
    }
}

void check_status(const char* name, sda_status_t s) {
    ++calls;
    if ((int)s < 0 || (int)s > 6) {
        std::fprintf(stderr, "%s returned status %d outside the enum\n", name, (int)s);
        std::exit(1);
    }
    ++errors_seen[(int)s];
    const char* msg = sda_last_error();
    const char* str = sda_status_string(s);
    if (!msg || !str || std::strlen(str) == 0) {
        std::fprintf(stderr, "%s: missing error string\n", name);
        std::exit(1);
    }
    (void)std::strlen(msg);
}

template <class... A>
void fuzz(const char* name, sda_status_t (*fn)(A...), int iters) {
    for (int i = 0; i < iters; ++i) {
        plausible = (i & 1) != 0;
        if (i % 64 == 0 || i % 64 == 1) reshuffle_layers();
        check_status(name, fn(draw<A>()...));
    }
}
template <class R, class... A>
void fuzz_size(const char* name, R (*fn)(A...), int iters) {
    for (int i = 0; i < iters; ++i) {
        plausible = (i & 1) != 0;
        volatile R r = fn(draw<A>()...);
        (void)r;
        ++calls;
    }
    (void)name;
}

// the chains read L host descriptors: keep L within the arrays the fuzzer owns
sda_status_t nsa_chain_bounded(const sda_nsa_layer* layers, const uint8_t* refresh, int L, const int32_t* seq_len,
                               int B, int NQ, int H_q, int H_kv, int d, int T_cap, int NC_cap, int cmp_stride,
                               int window, int top_n, int group_C, int mode, float scale, int32_t* bic,
                               int32_t* nsc, void* ws, size_t ws_bytes, void* stream) {
    L = L < -2 ? -2 : (L > kLayers ? kLayers : L);
    return sda_nsa_chain(layers, refresh, L, seq_len, B, NQ, H_q, H_kv, d, T_cap, NC_cap, cmp_stride, window, top_n,
                         group_C, mode, scale, bic, nsc, ws, ws_bytes, stream);
}
sda_status_t offload_chain_bounded(const sda_offload_layer* layers, int L, const int32_t* seq_len, int B, int H_q,
                                   int H_kv, int d, int T_cap, int n_init, int n_local, int top_k, float scale,
                                   const void* f_first, int pwg, int32_t* bio, void* ws, size_t ws_bytes,
                                   void* stream, void* side) {
    L = L < -2 ? -2 : (L > kLayers + 1 ? kLayers + 1 : L);      // one past the maximum: must be refused
    if (L > kLayers) return sda_offload_chain(layers, L, seq_len, B, H_q, H_kv, d, T_cap, n_init, n_local, top_k,
                                              scale, f_first, pwg, bio, ws, ws_bytes, stream, side) == SDA_OK
                               ? (sda_status_t)99 : SDA_ERR_SHAPE;
    return sda_offload_chain(layers, L, seq_len, B, H_q, H_kv, d, T_cap, n_init, n_local, top_k, scale, f_first,
                             pwg, bio, ws, ws_bytes, stream, side);
}

}  // namespace

int main(int argc, char** argv) {
    int n = 0;
    if (hipGetDeviceCount(&n) == hipSuccess && n > 0) {
        std::fprintf(stderr, "a GPU is visible: this fuzz passes host pointers as device buffers and must not run\n");
        return 3;
    }
    (void)hipGetLastError();
    const int iters = argc > 1 ? std::atoi(argv[1]) : 4000;
    for (int s = -3; s < 10; ++s) {
        const char* str = sda_status_string((sda_status_t)s);
        if (!str || std::strlen(str) == 0) {
            std::fprintf(stderr, "sda_status_string(%d) gave no text\n", s);
            return 1;
        }
    }
    (void)sda_version();
    fuzz("sda_update_compressed_keys", sda_update_compressed_keys, iters);
    fuzz("sda_update_compressed_keys_strided", sda_update_compressed_keys_strided, iters);
    fuzz_size("sda_score_select_workspace", sda_score_select_workspace, iters);
    fuzz("sda_score_select", sda_score_select, iters);
    fuzz_size("sda_score_select_multihead_workspace", sda_score_select_multihead_workspace, iters);
    fuzz("sda_score_select_multihead", sda_score_select_multihead, iters);
    fuzz_size("sda_score_select_multihead_pooled_workspace", sda_score_select_multihead_pooled_workspace, iters);
    fuzz("sda_score_select_multihead_pooled", sda_score_select_multihead_pooled, iters);
    fuzz_size("sda_score_select_pooled_workspace", sda_score_select_pooled_workspace, iters);
    fuzz("sda_score_select_pooled", sda_score_select_pooled, iters);
    fuzz_size("sda_sparse_decode_workspace", sda_sparse_decode_workspace, iters);
    fuzz("sda_sparse_decode", sda_sparse_decode, iters);
    fuzz_size("sda_grouped_decode_workspace", sda_grouped_decode_workspace, iters);
    fuzz("sda_grouped_decode", sda_grouped_decode, iters);
    fuzz_size("sda_nsa_decode_workspace", sda_nsa_decode_workspace, iters);
    fuzz("sda_nsa_decode", sda_nsa_decode, iters);
    fuzz_size("sda_nsa_chain_workspace", sda_nsa_chain_workspace, iters);
    fuzz("sda_nsa_chain", nsa_chain_bounded, iters);
    fuzz_size("sda_decode_step_workspace", sda_decode_step_workspace, iters);
    fuzz_size("sda_decode_step_is_fused", sda_decode_step_is_fused, iters);
    fuzz("sda_decode_step", sda_decode_step, iters);
    fuzz("sda_decode_step_noalloc", sda_decode_step_noalloc, iters);
    fuzz("sda_prefill_select", sda_prefill_select, iters);
    fuzz_size("sda_prefill_attention_workspace", sda_prefill_attention_workspace, iters);
    fuzz("sda_prefill_attention", sda_prefill_attention, iters);
    fuzz_size("sda_offload_chain_workspace", sda_offload_chain_workspace, iters);
    fuzz("sda_offload_chain", offload_chain_bounded, iters);
    fuzz("sda_gather_blocks", sda_gather_blocks, iters);
    std::printf("calls %lld; statuses ok %lld null %lld shape %lld unsupported %lld workspace %lld align %lld hip %lld\n",
                calls, errors_seen[0], errors_seen[1], errors_seen[2], errors_seen[3], errors_seen[4], errors_seen[5],
                errors_seen[6]);
    return 0;
}
