// spin_kv_quant kernel: head-wise Hadamard H_128 / sqrt(128) (R3, page
// "SpinQuant, Reproduced", Q5: the KV-path rotation runs online as a
// Hadamard) and INT4 KV-cache codes with one fp16 scale per (token, head)
// vector (abstract: 4-bit KV cache).
//
// Layout: one (token, head) vector of 128 values is owned by 16 lanes, 8
// consecutive values each (a 16-byte fp16 load per lane, fully coalesced).
// The three low index bits are butterflied in registers, the four high bits
// across the 16 lanes of a DPP row; the absmax is reduced across the same 16
// lanes.  Each lane then writes one dword of 8 packed codes, so a vector's 64
// code bytes are one contiguous 64-byte store.
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

constexpr int kKvThreads = 256;
constexpr int kKvGroupsPerBlock = kKvThreads / 16;

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float* v);

template <>
__device__ __forceinline__ void load8<__half>(const __half* p, float* v) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] & 0xFFFFu)));
        v[2 * i + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] >> 16)));
    }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename TIn, bool ROTATE, bool QUANT, bool WRITE_ROT>
__global__ __launch_bounds__(kKvThreads) void kv_quant_kernel(
    const TIn* __restrict__ X, long long groups, float norm, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scale, float* __restrict__ X_rot) {
    const long long g = static_cast<long long>(blockIdx.x) * kKvGroupsPerBlock + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    if (g >= groups) return;  // the 16 lanes of a vector leave together

    float v[8];
    load8<TIn>(X + g * 128 + l * 8, v);

    if (ROTATE) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] *= norm;
#pragma unroll
        for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j & h) continue;
                const float a = v[j];
                const float b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
#pragma unroll
        for (int msk = 1; msk < 16; msk <<= 1) {
            const bool upper = (l & msk) != 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = __shfl_xor(v[j], msk, 16);
                v[j] = upper ? (p - v[j]) : (v[j] + p);
            }
        }
    }

    if (WRITE_ROT) {
        float4* out = reinterpret_cast<float4*>(X_rot + g * 128 + l * 8);
        out[0] = make_float4(v[0], v[1], v[2], v[3]);
        out[1] = make_float4(v[4], v[5], v[6], v[7]);
    }

    if (QUANT) {
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[j]));
#pragma unroll
        for (int msk = 1; msk < 16; msk <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, msk, 16));
        const float s32 = __fdiv_rn(mx, kSeven);
        const __half s16 = __float2half_rn(s32);
        const float sf = __half2float(s16);
        int c8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c8[j] = quant_exact(v[j], sf);
        reinterpret_cast<uint32_t*>(codes)[g * 16 + l] = pack8(c8);
        if (l == 0) scale[g] = __half_as_ushort(s16);
    }
}

template <typename TIn, bool ROTATE, bool QUANT, bool WR>
hipError_t launch_kv_t(const TIn* X, long long groups, uint8_t* codes, uint16_t* scale,
                       float* Xr, hipStream_t s) {
    const float norm = static_cast<float>(1.0 / __builtin_sqrt(128.0));
    const long long blocks = (groups + kKvGroupsPerBlock - 1) / kKvGroupsPerBlock;
    hipLaunchKernelGGL((kv_quant_kernel<TIn, ROTATE, QUANT, WR>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kKvThreads), 0, s, X, groups, norm, codes, scale, Xr);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_kv_dispatch(const TIn* X, long long groups, bool rotate, uint8_t* codes,
                              uint16_t* scale, float* Xr, hipStream_t s) {
    const bool quant = codes != nullptr;
    const bool wr = Xr != nullptr;
    if (rotate) {
        if (quant) return wr ? launch_kv_t<TIn, true, true, true>(X, groups, codes, scale, Xr, s)
                             : launch_kv_t<TIn, true, true, false>(X, groups, codes, scale, Xr, s);
        return launch_kv_t<TIn, true, false, true>(X, groups, codes, scale, Xr, s);
    }
    if (quant) return wr ? launch_kv_t<TIn, false, true, true>(X, groups, codes, scale, Xr, s)
                         : launch_kv_t<TIn, false, true, false>(X, groups, codes, scale, Xr, s);
    return launch_kv_t<TIn, false, false, true>(X, groups, codes, scale, Xr, s);
}

}  // namespace

hipError_t launch_kv_quant(const void* X, bool x_f16, int T, int H, bool rotate, uint8_t* codes,
                           uint16_t* scale, float* X_rot, hipStream_t s) {
    const long long groups = static_cast<long long>(T) * H;
    if (x_f16)
        return launch_kv_dispatch<__half>(static_cast<const __half*>(X), groups, rotate, codes,
                                          scale, X_rot, s);
    return launch_kv_dispatch<float>(static_cast<const float*>(X), groups, rotate, codes, scale,
                                     X_rot, s);
}

}  // namespace spin
