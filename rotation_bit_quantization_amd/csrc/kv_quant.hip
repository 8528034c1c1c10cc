// spin_kv_quant kernel: head-wise Hadamard H_128 / sqrt(128) (R3, page
// "SpinQuant, Reproduced", Q5: the KV-path rotation runs online as a
// Hadamard) and INT4 KV-cache codes with one fp16 scale per (token, head)
// vector (abstract: 4-bit KV cache); BITS = 8 gives the KV8 variant (Q7 of the
// same page names W4A8KV8 among the evaluated settings), one byte per code.
//
// Layout: one (token, head) vector of 128 values is owned by 16 lanes, 8
// consecutive values each (a 16-byte fp16 load per lane, fully coalesced).
// The three low index bits are butterflied in registers, the four high bits
// across the 16 lanes of a DPP row (fused v_fmac_f32_dpp); the absmax is
// reduced across the same 16 lanes with DPP.  Each lane then writes one dword
// of 8 packed codes (two dwords of byte codes at 8 bits), so a vector's code
// bytes are one contiguous 64-byte (128-byte) store.  The normalisation 1/sqrt(128) is applied only where values are
// written or quantized (folded into the quantizer constant).
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

// Quantize eight held values z (true value = sign * z * norm) of one vector
// whose fp16 scale is s16: returns one dword of codes.  Fast path when s16 is
// a normal fp16 (then |y / s16| < 7.5 so no clamp is needed and the
// magic-number estimate plus exact near-tie fallback applies; 1/s16 from
// v_rcp_f32 keeps the estimate well inside the fallback window); otherwise the
// exact quotient and clamp.
__device__ __forceinline__ uint32_t kv_codes(const float* z, float sign, float norm, float sf) {
    if (sf >= 0x1p-14f && sf <= 65504.0f) {
        const float cr = sign * (norm * __builtin_amdgcn_rcpf(sf));
        uint32_t f[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = __float_as_uint(__builtin_fmaf(z[k], cr, kQuantMagic));
        const uint32_t m01 = min(f[0] & 0xFFFFu, f[1] & 0xFFFFu), m23 = min(f[2] & 0xFFFFu, f[3] & 0xFFFFu);
        const uint32_t m45 = min(f[4] & 0xFFFFu, f[5] & 0xFFFFu), m67 = min(f[6] & 0xFFFFu, f[7] & 0xFFFFu);
        if (min(min(m01, m23), min(m45, m67)) >= 3u) {
            const uint32_t ev = __builtin_amdgcn_perm(__builtin_amdgcn_perm(f[6], f[4], 0x0c0c0602u),
                                                      __builtin_amdgcn_perm(f[2], f[0], 0x0c0c0602u), 0x05040100u);
            const uint32_t od = __builtin_amdgcn_perm(__builtin_amdgcn_perm(f[7], f[5], 0x0c0c0602u),
                                                      __builtin_amdgcn_perm(f[3], f[1], 0x0c0c0602u), 0x05040100u);
            return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
        }
    }
    int c8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c8[k] = quant_exact((z[k] * sign) * norm, sf);
    return pack8(c8);
}

// The 8-bit variant of kv_codes: two dwords of byte codes.
__device__ __forceinline__ uint2 kv_codes8(const float* z, float sign, float norm, float sf) {
    if (sf >= 0x1p-14f && sf <= 65504.0f) {
        const float cr = sign * (norm * __builtin_amdgcn_rcpf(sf));
        uint32_t f[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = __float_as_uint(__builtin_fmaf(z[k], cr, kQuant8Magic));
        if (!any_near_tie8(f)) return make_uint2(pack4_magic8(f), pack4_magic8(f + 4));
    }
    int c8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c8[k] = quant_exact8((z[k] * sign) * norm, sf);
    return make_uint2(pack4b(c8), pack4b(c8 + 4));
}

// Two (token, head) vectors per 16-lane group: lane l holds values
// 8 g(l) .. 8 g(l) + 7 of each, g the DPP-basis load permutation, so that the
// four cross-lane butterfly levels (one v_fmac_f32_dpp each) leave lane l with
// values 8 l .. 8 l + 7 of the transform times (-1)^popcount(l & 7).  The
// first in-register level reads both fp16 halves with a mixed-precision FMA
// (`one` = 1.0 passed at run time keeps it an FMA).
// `block` is the workgroup's index within the tensor X.
template <int BITS, typename TIn, bool ROTATE, bool QUANT, bool WRITE_ROT>
__device__ __forceinline__ void kv_vectors(const TIn* __restrict__ X, long long groups, float norm, float one,
                                           uint8_t* __restrict__ codes, uint16_t* __restrict__ scale,
                                           float* __restrict__ X_rot, long long block) {
    constexpr int kPer = 2;
    const int l = threadIdx.x & 15;
    const long long g0 = (block * kKvGroupsPerBlock + (threadIdx.x >> 4)) * kPer;
    if (g0 >= groups) return;  // the 16 lanes of a group leave together
    const int src = ROTATE ? g_perm(l) : l;

    float v[kPer][8];
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
        const long long g = g0 + p < groups ? g0 + p : g0;
        if (sizeof(TIn) == 2) {
            const uint4 raw = *reinterpret_cast<const uint4*>(X + g * 128 + src * 8);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
            if (ROTATE) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {   // level over index bit 0, straight from fp16
                    const float lo = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] & 0xFFFFu)));
                    const float hi = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] >> 16)));
                    v[p][2 * i] = __builtin_fmaf(lo, one, hi);
                    v[p][2 * i + 1] = __builtin_fmaf(hi, -one, lo);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[p][2 * i] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] & 0xFFFFu)));
                    v[p][2 * i + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] >> 16)));
                }
            }
        } else {
            load8<TIn>(X + g * 128 + src * 8, v[p]);
            if (ROTATE) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a = v[p][2 * i], b = v[p][2 * i + 1];
                    v[p][2 * i] = a + b;
                    v[p][2 * i + 1] = a - b;
                }
            }
        }
    }
    float sign = 1.0f;
    if (ROTATE) {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
#pragma unroll
            for (int h = 2; h < 8; h <<= 1) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (j & h) continue;
                    const float a = v[p][j];
                    const float b = v[p][j + h];
                    v[p][j] = a + b;
                    v[p][j + h] = a - b;
                }
            }
        }
        dpp_wht16<16>(&v[0][0], lane_sign(l, 0b0101), lane_sign(l, 0b0110), lane_sign(l, 0b1100),
                      lane_sign(l, 0b1000));
        sign = lane_sign(l, 0b0111);
    }
    const float nrm = ROTATE ? norm : 1.0f;

#pragma unroll
    for (int p = 0; p < kPer; ++p) {
        const long long g = g0 + p;
        if (g >= groups) break;
        if (WRITE_ROT) {
            float y[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = (v[p][k] * sign) * nrm;
            float4* out = reinterpret_cast<float4*>(X_rot + g * 128 + l * 8);
            out[0] = make_float4(y[0], y[1], y[2], y[3]);
            out[1] = make_float4(y[4], y[5], y[6], y[7]);
        }
        if (QUANT) {
            float mx = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[p][k]));
            mx = row16_max(mx) * nrm;                 // = max_i fl32(|z_i| * norm)
            // Any absmax above 65504 * 7 rounds to an fp16 infinity; clamping
            // at 2^100 keeps that result for an infinite absmax, whose
            // remainder step in div_by_qmax would otherwise give NaN.
            mx = __builtin_fminf(mx, 0x1p100f);
            const __half s16 = __float2half_rn(BITS == 4 ? div_by_qmax(mx, kSeven, kRcpSeven)
                                                          : div_by_qmax(mx, kQmax8, kRcpQmax8));
            const float sf = __half2float(s16);
            if (BITS == 4)
                reinterpret_cast<uint32_t*>(codes)[g * 16 + l] = kv_codes(v[p], sign, nrm, sf);
            else
                reinterpret_cast<uint2*>(codes)[g * 16 + l] = kv_codes8(v[p], sign, nrm, sf);
            if (l == 0) scale[g] = __half_as_ushort(s16);
        }
    }
}

template <int BITS, typename TIn, bool ROTATE, bool QUANT, bool WRITE_ROT>
__global__ __launch_bounds__(kKvThreads) void kv_quant_kernel(
    const TIn* __restrict__ X, long long groups, float norm, float one, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scale, float* __restrict__ X_rot) {
    kv_vectors<BITS, TIn, ROTATE, QUANT, WRITE_ROT>(X, groups, norm, one, codes, scale, X_rot, blockIdx.x);
}

// The KV step of one attention layer: the grid's first bk workgroups take K
// (rotated and quantized), the next bv take V (quantized only), the rest Q
// (rotated only).  Each workgroup runs exactly the code of the matching
// single-tensor kernel, so the outputs are the same bits.
struct KvQkvArgs {
    const void* Q;
    const void* K;
    const void* V;
    long long gq, gk, gv;          // (token, head) vectors per tensor
    long long bk, bv;              // workgroups of K and of V
    float norm, one;
    float* Q_rot;
    uint8_t* K_codes;
    uint16_t* K_scale;
    float* K_rot;
    uint8_t* V_codes;
    uint16_t* V_scale;
};

template <int BITS, typename TIn, bool K_ROT>
__global__ __launch_bounds__(kKvThreads) void kv_qkv_kernel(KvQkvArgs a) {
    const long long b = blockIdx.x;
    if (b < a.bk)
        kv_vectors<BITS, TIn, true, true, K_ROT>(static_cast<const TIn*>(a.K), a.gk, a.norm, a.one, a.K_codes,
                                                 a.K_scale, a.K_rot, b);
    else if (b < a.bk + a.bv)
        kv_vectors<BITS, TIn, false, true, false>(static_cast<const TIn*>(a.V), a.gv, a.norm, a.one, a.V_codes,
                                                  a.V_scale, nullptr, b - a.bk);
    else
        kv_vectors<BITS, TIn, true, false, true>(static_cast<const TIn*>(a.Q), a.gq, a.norm, a.one, nullptr,
                                                 nullptr, a.Q_rot, b - a.bk - a.bv);
}

template <int BITS, typename TIn, bool ROTATE, bool QUANT, bool WR>
hipError_t launch_kv_t(const TIn* X, long long groups, uint8_t* codes, uint16_t* scale,
                       float* Xr, hipStream_t s) {
    const float norm = static_cast<float>(1.0 / __builtin_sqrt(128.0));
    const long long per_block = 2LL * kKvGroupsPerBlock;
    const long long blocks = (groups + per_block - 1) / per_block;
    hipLaunchKernelGGL((kv_quant_kernel<BITS, TIn, ROTATE, QUANT, WR>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kKvThreads), 0, s, X, groups, norm, 1.0f, codes, scale, Xr);
    return hipGetLastError();
}

template <int BITS, typename TIn>
hipError_t launch_kv_dispatch(const TIn* X, long long groups, bool rotate, uint8_t* codes,
                              uint16_t* scale, float* Xr, hipStream_t s) {
    const bool quant = codes != nullptr;
    const bool wr = Xr != nullptr;
    if (rotate) {
        if (quant) return wr ? launch_kv_t<BITS, TIn, true, true, true>(X, groups, codes, scale, Xr, s)
                             : launch_kv_t<BITS, TIn, true, true, false>(X, groups, codes, scale, Xr, s);
        return launch_kv_t<BITS, TIn, true, false, true>(X, groups, codes, scale, Xr, s);
    }
    if (quant) return wr ? launch_kv_t<BITS, TIn, false, true, true>(X, groups, codes, scale, Xr, s)
                         : launch_kv_t<BITS, TIn, false, true, false>(X, groups, codes, scale, Xr, s);
    return launch_kv_t<BITS, TIn, false, false, true>(X, groups, codes, scale, Xr, s);
}

template <int BITS>
hipError_t launch_kv_bits(const void* X, bool x_f16, long long groups, bool rotate, uint8_t* codes,
                          uint16_t* scale, float* X_rot, hipStream_t s) {
    if (x_f16)
        return launch_kv_dispatch<BITS, __half>(static_cast<const __half*>(X), groups, rotate, codes,
                                                scale, X_rot, s);
    return launch_kv_dispatch<BITS, float>(static_cast<const float*>(X), groups, rotate, codes, scale,
                                           X_rot, s);
}

template <int BITS, typename TIn>
hipError_t launch_kv_qkv_t(const KvQkvArgs& a, long long blocks, hipStream_t s) {
    if (a.K_rot)
        hipLaunchKernelGGL((kv_qkv_kernel<BITS, TIn, true>), dim3(static_cast<unsigned>(blocks)), dim3(kKvThreads),
                           0, s, a);
    else
        hipLaunchKernelGGL((kv_qkv_kernel<BITS, TIn, false>), dim3(static_cast<unsigned>(blocks)), dim3(kKvThreads),
                           0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_qkv(const void* Q, const void* K, const void* V, bool x_f16, int T, int Hq, int Hkv,
                         int bits, float* Q_rot, uint8_t* K_codes, uint16_t* K_scale, float* K_rot,
                         uint8_t* V_codes, uint16_t* V_scale, hipStream_t s) {
    const long long per_block = 2LL * kKvGroupsPerBlock;
    KvQkvArgs a;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.gq = Q ? static_cast<long long>(T) * Hq : 0;
    a.gk = a.gv = static_cast<long long>(T) * Hkv;
    a.bk = a.bv = (a.gk + per_block - 1) / per_block;
    a.norm = static_cast<float>(1.0 / __builtin_sqrt(128.0));
    a.one = 1.0f;
    a.Q_rot = Q_rot;
    a.K_codes = K_codes;
    a.K_scale = K_scale;
    a.K_rot = K_rot;
    a.V_codes = V_codes;
    a.V_scale = V_scale;
    const long long blocks = a.bk + a.bv + (a.gq + per_block - 1) / per_block;
    if (blocks == 0) return hipSuccess;
    if (bits == 8)
        return x_f16 ? launch_kv_qkv_t<8, __half>(a, blocks, s) : launch_kv_qkv_t<8, float>(a, blocks, s);
    return x_f16 ? launch_kv_qkv_t<4, __half>(a, blocks, s) : launch_kv_qkv_t<4, float>(a, blocks, s);
}

hipError_t launch_kv_quant(const void* X, bool x_f16, int T, int H, bool rotate, int bits, uint8_t* codes,
                           uint16_t* scale, float* X_rot, hipStream_t s) {
    const long long groups = static_cast<long long>(T) * H;
    // rotate-only calls (no codes) are the same for either width
    return bits == 8 && codes ? launch_kv_bits<8>(X, x_f16, groups, rotate, codes, scale, X_rot, s)
                              : launch_kv_bits<4>(X, x_f16, groups, rotate, codes, scale, X_rot, s);
}

}  // namespace spin
