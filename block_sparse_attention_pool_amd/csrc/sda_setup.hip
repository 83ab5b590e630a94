// Per-device set-up of libsda, done once per device at the first call of any
// entry point on it, and the scratch array of the no-allocation decode step.
// Set-up records are written under a lock and never change afterwards;
// nothing in them changes a call's results.
#include <atomic>
#include <mutex>

#include "sda_internal.h"

namespace sda {

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_setup_lock;
std::atomic<bool> g_ready[kMaxDevices];

// Scratch of sda_decode_step_noalloc: one copy per device, held until the
// process ends.  The first kNoallocCounterBytes hold arrival counters (zero
// between calls: every completed call resets the ones it used); split
// partials, scores and candidate lists follow.  Host code never names this
// array after set-up: it uses the device address recorded per device.
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::atomic<bool> g_scratch_ready[kMaxDevices];
char* g_scratch_ptr[kMaxDevices];

__global__ void zero_words(uint32_t* p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t current_device(int* dev) {
    const hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return e;
    return (*dev < 0 || *dev >= kMaxDevices) ? hipErrorInvalidDevice : hipSuccess;
}

}  // namespace

hipError_t device_setup() {
    int dev = 0;
    hipError_t e = current_device(&dev);
    if (e != hipSuccess) return e;
    if (g_ready[dev].load(std::memory_order_acquire)) return hipSuccess;
    std::lock_guard<std::mutex> guard(g_setup_lock);
    if (g_ready[dev].load(std::memory_order_relaxed)) return hipSuccess;
    e = attn_grant_lds();
    if (e == hipSuccess) e = tiled_grant_lds();
    if (e != hipSuccess) return e;
    g_ready[dev].store(true, std::memory_order_release);
    return hipSuccess;
}

hipError_t noalloc_scratch(hipStream_t s, char** ptr) {
    int dev = 0;
    hipError_t e = current_device(&dev);
    if (e != hipSuccess) return e;
    if (!g_scratch_ready[dev].load(std::memory_order_acquire)) {
        std::lock_guard<std::mutex> guard(g_setup_lock);
        if (!g_scratch_ready[dev].load(std::memory_order_relaxed)) {
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            // static storage starts zero-filled; the counter region is cleared
            // once more by a fill kernel on the caller's stream, ahead of the
            // first call's launch
            hipLaunchKernelGGL(zero_words, dim3(16), dim3(256), 0, s, static_cast<uint32_t*>(p),
                               kNoallocCounterBytes / sizeof(uint32_t));
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            g_scratch_ptr[dev] = static_cast<char*>(p);
            g_scratch_ready[dev].store(true, std::memory_order_release);
        }
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace sda
