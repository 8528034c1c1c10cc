// Machine probes for the benchmark report (libspin_probe, not part of
// libspin): the sustained dense MFMA rate of the two instructions the hot path
// uses, the shader clock while the matrix cores are busy, and the streaming
// read bandwidth of HBM.  They give the measured ceilings that the kernels'
// roofline fractions can be read against, beside the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spin_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;

// Each wave runs `iters` rounds of four independent MFMA chains on operands
// taken from `operands` (8 dwords per lane: A in dwords 0-3, B in 4-7), so that
// the matrix cores see data of the hot path's kind rather than constants.
// Lane 0 of every wave records its start and end in shader cycles and in the
// constant 100 MHz real-time counter.
template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void probe_mfma(const uint32_t* __restrict__ operands, int iters,
                                                            int64_t* __restrict__ timing) {
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
    const u4v a = *reinterpret_cast<const u4v*>(operands + 8 * lane);
    const u4v b = *reinterpret_cast<const u4v*>(operands + 8 * lane + 4);
    const int64_t c0 = static_cast<int64_t>(__builtin_readcyclecounter());
    const int64_t r0 = static_cast<int64_t>(__builtin_amdgcn_s_memrealtime());
    int check = 0;
    if (KIND == 0) {
        const v4i av = __builtin_bit_cast(v4i, a), bv = __builtin_bit_cast(v4i, b);
        v16i acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
        for (int i = 0; i < iters; ++i) {
            acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(bv, av, acc1, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, av, acc2, 0, 0, 0);
            acc3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(bv, bv, acc3, 0, 0, 0);
        }
        check = acc0[0] ^ acc1[5] ^ acc2[10] ^ acc3[15];
    } else {
        const h8v av = __builtin_bit_cast(h8v, a), bv = __builtin_bit_cast(h8v, b);
        f16v acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
        for (int i = 0; i < iters; ++i) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv, av, acc1, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, av, acc2, 0, 0, 0);
            acc3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv, bv, acc3, 0, 0, 0);
        }
        check = __float_as_int(acc0[0] + acc1[5] + acc2[10] + acc3[15]);
    }
    const int64_t c1 = static_cast<int64_t>(__builtin_readcyclecounter());
    const int64_t r1 = static_cast<int64_t>(__builtin_amdgcn_s_memrealtime());
    if (lane == 0) {
        int64_t* t = timing + 4 * static_cast<size_t>(wave);
        t[0] = c0;
        t[1] = c1;
        t[2] = r0;
        // the accumulators are folded into the last word so that no chain is dead
        t[3] = r1 + (check == 0x7F7F7F7F ? 1 : 0);
    }
}

// Grid-stride streaming read of `n16` 16-byte words with non-temporal loads;
// the sum is stored only under a condition the data never meets.
__global__ __launch_bounds__(kProbeThreads) void probe_read(const u4v* __restrict__ buf, size_t n16,
                                                            uint32_t* __restrict__ sink) {
    constexpr int kUnroll = 4;
    uint32_t acc = 0;
    const size_t stride = static_cast<size_t>(gridDim.x) * kProbeThreads * kUnroll;
    for (size_t base = static_cast<size_t>(blockIdx.x) * kProbeThreads * kUnroll + threadIdx.x; base < n16;
         base += stride) {
        u4v r[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t i = base + static_cast<size_t>(u) * kProbeThreads;
            r[u] = i < n16 ? __builtin_nontemporal_load(buf + i) : u4v{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= r[u][0] + r[u][1] + r[u][2] + r[u][3];
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" spin_status spin_probe_mfma(int kind, int blocks, int iters, const uint32_t* operands, int64_t* timing,
                                       void* stream) {
    if (!operands || !timing) return SPIN_ERR_NULL;
    if ((kind != 0 && kind != 1) || blocks <= 0 || blocks > (1 << 20) || iters <= 0 || iters > (1 << 24))
        return SPIN_ERR_BAD_SHAPE;
    if ((reinterpret_cast<uintptr_t>(operands) & 15u) || (reinterpret_cast<uintptr_t>(timing) & 15u))
        return SPIN_ERR_MISALIGNED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind == 0)
        hipLaunchKernelGGL(probe_mfma<0>, dim3(blocks), dim3(kProbeThreads), 0, s, operands, iters, timing);
    else
        hipLaunchKernelGGL(probe_mfma<1>, dim3(blocks), dim3(kProbeThreads), 0, s, operands, iters, timing);
    return hipGetLastError() == hipSuccess ? SPIN_OK : SPIN_ERR_HIP;
}

extern "C" spin_status spin_probe_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, void* stream) {
    if (!buf || !sink) return SPIN_ERR_NULL;
    if (bytes == 0 || (bytes & 15u) || blocks <= 0 || blocks > (1 << 20)) return SPIN_ERR_BAD_SHAPE;
    if (reinterpret_cast<uintptr_t>(buf) & 15u) return SPIN_ERR_MISALIGNED;
    hipLaunchKernelGGL(probe_read, dim3(blocks), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u4v*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? SPIN_OK : SPIN_ERR_HIP;
}
