// Device helpers shared by the INT4-weight GEMM kernels (W4A4 and W4A8):
// the INT4 -> INT8 widening of packed weight codes, the LDS DMA issue and its
// waits, the LDS slot swizzle of 64-byte operand rows, and the XCD-aware tile
// order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spin_device.h"

namespace spin {

// Sixteen packed nibbles (one uint2) -> sixteen int8 lanes holding 16 * code:
// bytes {c0, c2, c4, c6}, {c1, c3, c5, c7}, {c8, ..., c14}, {c9, ..., c15} (codes
// numbered from the low nibble of the first byte).  Masking with 0xF0F0F0F0
// keeps the odd codes in the high nibble of each byte; a left shift by 4 first
// does the same for the even codes.  Both GEMM operands must present their k
// values in this same order.
__device__ __forceinline__ v4i widen16(uint2 p) {
    v4i r;
    r.x = static_cast<int>((p.x << 4) & 0xF0F0F0F0u);
    r.y = static_cast<int>(p.x & 0xF0F0F0F0u);
    r.z = static_cast<int>((p.y << 4) & 0xF0F0F0F0u);
    r.w = static_cast<int>(p.y & 0xF0F0F0F0u);
    return r;
}

typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void tile_of(int bid, int tilesM, int tilesN, int* tm, int* tn) {
    const int T = tilesM * tilesN;
    int t = bid;
    if ((T & 7) == 0) t = (bid & 7) * (T >> 3) + (bid >> 3);    // contiguous block per XCD
    constexpr int G = 4;                                        // tile rows per group
    const int group = t / (G * tilesN);
    const int first = group * G;
    const int rows = min(G, tilesM - first);
    const int r = t - group * G * tilesN;
    *tm = first + r % rows;
    *tn = r / rows;
}

// After the main loop: once every wave has left it (the first barrier; no
// stage is read or filled after that), every thread with `has` set stores
// `v` to word threadIdx.x of the LDS, and the workgroup waits; returns the
// words as floats.
__device__ __forceinline__ const float* stage_scales(uint8_t* lds, float v, bool has) {
    float* sc = reinterpret_cast<float*>(lds);
    __syncthreads();
    if (has) sc[threadIdx.x] = v;
    __syncthreads();
    return sc;
}

__device__ __forceinline__ int slot_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

typedef const __attribute__((address_space(3))) void* lds_cptr;

// Byte offset of a __shared__ object within the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cptr)(p)));
}

// s_waitcnt with only the vector-memory counter limited to n (n < 16).
#define SPIN_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((n) | 0x0F70)

// Workgroup barrier that is also a compiler memory barrier (no load or store
// moves across it) but, unlike __syncthreads, not a memory fence: it does not
// wait for the LDS-DMA loads still in flight for later steps.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from `src` into LDS at byte address lds_base + 16 * lane
// (lds_base wave-uniform).  M0 is saved and restored around it, with the one
// wait state an LDS DMA needs after an SALU write of M0; the only register
// operand is the address, which the load consumes at issue.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds_base)
        : "memory");
}

}  // namespace spin
