// Per-device set-up of libsda, done once per device at the first call of any
// entry point on it.  The record is written under a lock and never changes
// afterwards; nothing in it changes a call's results.
#include <atomic>
#include <mutex>

#include "sda_internal.h"

namespace sda {

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_setup_lock;
std::atomic<bool> g_ready[kMaxDevices];

}  // namespace

hipError_t device_setup() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (g_ready[dev].load(std::memory_order_acquire)) return hipSuccess;
    std::lock_guard<std::mutex> guard(g_setup_lock);
    if (g_ready[dev].load(std::memory_order_relaxed)) return hipSuccess;
    e = attn_grant_lds();
    if (e != hipSuccess) return e;
    g_ready[dev].store(true, std::memory_order_release);
    return hipSuccess;
}

}  // namespace sda
