// Pieces shared by the attention kernels: the token order of the QK tile,
// the LDS layout of a V tile read back transposed, direct-to-LDS loads and
// read-only scalar reads.
#pragma once
#include <stdint.h>

#include "sda_device.hpp"
#include "sda_internal.h"

namespace sda {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4i16;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
#define SDA_LDS __attribute__((address_space(3)))

// token held in QK A-operand row m of m-tile mt
__device__ __forceinline__ int tok_of(int mt, int m) {
    return (mt >> 1) * 32 + (m >> 2) * 8 + (mt & 1) * 4 + (m & 3);
}

// A V tile in LDS: 64 rows of d bf16.  The 32-byte chunks of row
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

// Read-only int32 the kernel never writes (lengths, block lists): through the
// constant address space, so that wave-uniform reads become scalar loads
// that wait on their own counter, not behind the vector loads.
__device__ __forceinline__ int ld_ro(const int32_t* p) {
    return *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)p;
}

template <int AUX = 0>
__device__ __forceinline__ void lds_dma16(const void* g, SDA_LDS void* l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, AUX);
}

// The same direct load, issued as assembly: the compiler then does not know
// that it writes LDS, so it adds no wait for it before later LDS reads (it
// would wait for every direct load in flight, the prefetched blocks
// included); the caller waits for it with an explicit vmcnt wait.  M0 holds
// the wave-uniform LDS address (one wait state between setting M0 and the
// load).
__device__ __forceinline__ void lds_dma16_async(const void* g, SDA_LDS void* l) {
    const uint32_t m = (uint32_t)(uintptr_t)l;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}

// A workgroup barrier that waits for this wave's LDS operations but not for
// its vector memory loads (the direct loads of later blocks stay in flight).
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace sda
