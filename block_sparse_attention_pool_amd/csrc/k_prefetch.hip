// Persistent prefetch pool for offloaded K/V ([SparDA] §4.5 and fig. 5: a
// small set of long-lived workgroups waits for transfer requests for the
// whole decode; when layer l has chosen the blocks of layer l+1, the main
// stream enqueues the request and goes on with layer l's attention while the
// pool copies the blocks from pinned host memory into a device stage; layer
// l+1's attention waits for the request's completion, §4.2 steps 3 and 6).
//
// Control words (device, zeroed before the pool starts):
//   ctrl[kTail]          requests enqueued so far (request r = layer r)
//   ctrl[kStop]          set by the main stream when the chain ends
//   ctrl[kError]         1: a pool workgroup gave up waiting for a request;
//                        2: a waiter gave up waiting for a request's completion
//   ctrl[kClaim + r]     next block task of request r to hand out
//   ctrl[kDone + r]      block tasks of request r completed
// Every wait is bounded (spin_limit polls with a sleep between them), so
// every workgroup exits even if a request never comes.  Pool workgroups
// claim block tasks one at a time; each task copies one selected block (its
// K and V rows) with agent-scope (write-through) stores, waits for them to
// complete, and then counts itself done, so a waiter that sees the full
// count (with an acquire load) finds every block of the stage in place.
#include <algorithm>

#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

namespace {

__device__ __forceinline__ int ld_acq(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_rlx(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rlx(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// a 16-byte chunk as two agent-scope 64-bit stores
__device__ __forceinline__ void st16_wt(uint16_t* dst, const u32x4& v) {
    uint64_t* p = reinterpret_cast<uint64_t*>(dst);
    __hip_atomic_store(p, ((uint64_t)v[1] << 32) | v[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 1, ((uint64_t)v[3] << 32) | v[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
__global__ __launch_bounds__(256) void prefetch_pool_kernel(PrefetchArgs a) {
    constexpr int CHUNKS = kBlock * D / 8;     // 16-byte chunks per block
    constexpr int CPR = D / 8;                 // chunks per token row
    __shared__ int s_go, s_task;
    int* ctrl = a.ctrl;
    const int total = a.rows * a.n_sel_max;
    for (int r = 0; r < a.L; ++r) {
        if (threadIdx.x == 0) {
            int go = 0;
            for (int it = 0; it < a.spin_limit; ++it) {
                if (ld_acq(ctrl + kPfTail) > r) {
                    go = 1;
                    break;
                }
                if (ld_rlx(ctrl + kPfStop)) break;
                __builtin_amdgcn_s_sleep(127);
            }
            if (!go && !ld_rlx(ctrl + kPfStop)) st_rlx(ctrl + kPfError, 1);
            s_go = go;
        }
        __syncthreads();
        if (!s_go) return;                      // uniform: stopped, or no request came
        const PrefetchLayer& y = a.layer[r];
        for (;;) {
            if (threadIdx.x == 0)
                s_task = __hip_atomic_fetch_add(ctrl + kPfClaim + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const int task = s_task;
            __syncthreads();                    // s_task is rewritten by the next claim
            if (task >= total) break;
            const int row = task / a.n_sel_max;
            const int e = task - row * a.n_sel_max;
            const int n = y.n_sel[row];
            const int j = (e < n) ? y.block_idx[(size_t)row * a.n_sel_max + e] : -1;
            const bool ok = (e < n) && j >= 0 && (size_t)j * kBlock < (size_t)a.T_cap;
            if (threadIdx.x == 0) st_rlx(y.slot + (size_t)row * a.n_sel_max + e, ok ? e : -1);
            if (ok) {
                const int rows_avail = min(kBlock, a.T_cap - j * kBlock);
                const size_t src = ((size_t)row * a.T_cap + (size_t)j * kBlock) * D;
                const size_t dst = ((size_t)row * a.n_sel_max * kBlock + (size_t)e * kBlock) * D;
                u32x4 kr[CHUNKS / 256], vr[CHUNKS / 256];
#pragma unroll
                for (int i = 0; i < CHUNKS / 256; ++i) {
                    const int c = threadIdx.x + i * 256;
                    if (c / CPR < rows_avail) {
                        kr[i] = ldg16(y.k_src + src + (size_t)c * 8);
                        vr[i] = ldg16(y.v_src + src + (size_t)c * 8);
                    } else {
                        kr[i] = u32x4{0, 0, 0, 0};
                        vr[i] = u32x4{0, 0, 0, 0};
                    }
                }
#pragma unroll
                for (int i = 0; i < CHUNKS / 256; ++i) {
                    const int c = threadIdx.x + i * 256;
                    st16_wt(y.k_stage + dst + (size_t)c * 8, kr[i]);
                    st16_wt(y.v_stage + dst + (size_t)c * 8, vr[i]);
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's stores are visible
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(ctrl + kPfDone + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// request r is enqueued: the layer's block lists were written by earlier
// launches on this stream
__global__ void prefetch_enqueue_kernel(int* ctrl, int r) {
    if (threadIdx.x == 0) __hip_atomic_store(ctrl + kPfTail, r + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// the stream waits (one wave, bounded) until every block task of request r is done
__global__ void prefetch_wait_kernel(int* ctrl, int r, int total, int spin_limit) {
    if (threadIdx.x != 0) return;
    for (int it = 0; it < spin_limit; ++it) {
        if (ld_acq(ctrl + kPfDone + r) >= total) return;
        if (ld_rlx(ctrl + kPfError)) return;    // the pool gave up: stop waiting too
        __builtin_amdgcn_s_sleep(127);
    }
    st_rlx(ctrl + kPfError, 2);
}

__global__ void prefetch_stop_kernel(int* ctrl) {
    if (threadIdx.x == 0) st_rlx(ctrl + kPfStop, 1);
}

__global__ void zero_ints_kernel(int* p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

}  // namespace

hipError_t launch_prefetch_reset(int* ctrl, hipStream_t s) {
    hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(256), 0, s, ctrl, (size_t)kPfCtrlInts);
    return hipGetLastError();
}

hipError_t launch_zero_words(void* p, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_ints_kernel, dim3(grid), dim3(256), 0, s, static_cast<int*>(p), n);
    return hipGetLastError();
}

hipError_t launch_prefetch_pool(const PrefetchArgs& a, int d, int workgroups, hipStream_t s) {
    if (d == 128) hipLaunchKernelGGL(prefetch_pool_kernel<128>, dim3(workgroups), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(prefetch_pool_kernel<64>, dim3(workgroups), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prefetch_enqueue(int* ctrl, int r, hipStream_t s) {
    hipLaunchKernelGGL(prefetch_enqueue_kernel, dim3(1), dim3(64), 0, s, ctrl, r);
    return hipGetLastError();
}

hipError_t launch_prefetch_wait(int* ctrl, int r, int total, int spin_limit, hipStream_t s) {
    hipLaunchKernelGGL(prefetch_wait_kernel, dim3(1), dim3(64), 0, s, ctrl, r, total, spin_limit);
    return hipGetLastError();
}

hipError_t launch_prefetch_stop(int* ctrl, hipStream_t s) {
    hipLaunchKernelGGL(prefetch_stop_kernel, dim3(1), dim3(64), 0, s, ctrl);
    return hipGetLastError();
}

}  // namespace sda
