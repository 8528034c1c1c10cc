// spin_fwht_quant kernels: online Hadamard of each activation row followed by
// per-token symmetric INT4 (page "SpinQuant, Reproduced", Q5: R4 before
// down_proj runs online as a Hadamard over the MLP width; abstract: 4-bit
// activations).  Every kernel is templated on the code width BITS: 4 (codes
// packed two per byte, scale max|y| / 7) or 8 (the W4A8 variant the same page
// lists in Q7: one signed byte per code, scale max|y| / 127); only the
// quantizer epilogue differs.
//
// fwht_quant_rowlds: one workgroup per row; the row is staged in LDS as
// float32, normalised by fl32(1/sqrt(n)) on load, transformed by radix-2
// butterflies over the power-of-two index bits (one LDS pass per level), then
// by the order-12 mix across the 12 sub-blocks when n = 12 * 2^k, reduced to
// its absmax, quantized with the exact IEEE quotient and packed.  It serves
// every supported order and row length.
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

constexpr int kRowThreads = 256;

template <int BITS, typename TIn, bool WRITE_ROT>
__global__ __launch_bounds__(kRowThreads) void fwht_quant_rowlds(
    const TIn* __restrict__ X, int K, int log2p, int has12, int rotate, float norm,
    uint8_t* __restrict__ Xq, float* __restrict__ x_scale, float* __restrict__ X_rot) {
    extern __shared__ float row[];
    __shared__ float red[4];
    const size_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const TIn* xr = X + m * static_cast<size_t>(K);

    for (int i = tid; i < K; i += kRowThreads) row[i] = load_as_float(xr + i) * norm;
    __syncthreads();

    if (rotate) {
        // Sylvester levels: pair (i, i + h) for every i with bit h clear.
        for (int l = 0; l < log2p; ++l) {
            const int h = 1 << l;
            for (int t = tid; t < K / 2; t += kRowThreads) {
                const int i = ((t >> l) << (l + 1)) | (t & (h - 1));
                const float a = row[i];
                const float b = row[i + h];
                row[i] = a + b;
                row[i + h] = a - b;
            }
            __syncthreads();
        }
        if (has12) {
            // y_c = sum_a H12[a][c] z_a over the 12 sub-blocks of each block.
            const int P = 1 << log2p;
            for (int col = tid; col < K / 12; col += kRowThreads) {
                const int blk = col >> log2p;
                const int b = col & (P - 1);
                const int base = blk * 12 * P + b;
                float z[12];
#pragma unroll
                for (int a = 0; a < 12; ++a) z[a] = row[base + a * P];
#pragma unroll
                for (int c = 0; c < 12; ++c) {
                    float acc = 0.0f;
#pragma unroll
                    for (int a = 0; a < 12; ++a) acc += h12_sign(a, c) * z[a];
                    row[base + c * P] = acc;
                }
            }
            __syncthreads();
        }
    }

    float mx = 0.0f;
    for (int i = tid; i < K; i += kRowThreads) mx = __builtin_fmaxf(mx, __builtin_fabsf(row[i]));
    const float amax = block_max_256(mx, red);
    const float s = __fdiv_rn(amax, BITS == 4 ? kSeven : kQmax8);
    if (tid == 0) x_scale[m] = s;

    uint8_t* out = Xq + m * static_cast<size_t>(BITS == 4 ? K / 2 : K);
    for (int g = tid; g < K / 8; g += kRowThreads) {
        int c8[8];
        if (BITS == 4) {
#pragma unroll
            for (int j = 0; j < 8; ++j) c8[j] = quant_exact(row[8 * g + j], s);
            reinterpret_cast<uint32_t*>(out)[g] = pack8(c8);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) c8[j] = quant_exact8(row[8 * g + j], s);
            reinterpret_cast<uint2*>(out)[g] = make_uint2(pack4b(c8), pack4b(c8 + 4));
        }
    }
    if (WRITE_ROT) {
        float* yr = X_rot + m * static_cast<size_t>(K);
        for (int i = tid; i < K; i += kRowThreads) yr[i] = row[i];
    }
}

// ---------------------------------------------------------------------------
// fwht_quant_k12288: the R4 / down_proj case, fp16 rows of 12288 = 12 x 1024
// with had_n = 12288.  Element i = a * 1024 + b; the transform is
// Y = H12^T X H1024 on the 12 x 1024 view (x . (H12 (x) H1024)).
//
// One workgroup of 256 threads per row, two register layouts and one LDS
// exchange:
//   phase 1  thread holds x[a][4 beta + j] for all 12 a and j = 0..3
//            (twelve 8-byte loads).  b bits 0-1 are butterflied in registers,
//            the H12 mix runs in registers, b bits 2-5 are the low lane bits
//            (four DPP levels); b bits 6-7 are lane bits 4-5, b bits 8-9 the
//            wave.
//   LDS      the rotated values are written in natural order, 64-float rows
//            padded to 68 so that the phase-2 reads spread over the banks; the
//            exchange runs in two rounds of six a each (26 KB of LDS per
//            workgroup instead of 52 KB, so twice as many workgroups fit a CU).
//   phase 2  thread holds 8 consecutive b (bits 0-2) for 6 of the 12 a: b bits
//            6-9 are the low lane bits (four more DPP levels), b bits 3-4 lane
//            bits 4-5, b bit 5 wave bit 0, the half of a wave bit 1.
// Each DPP stage leaves lane i with (-1)^popcount(i & 7) times its value; both
// signs, and nothing else, are folded into the per-thread quantizer constant.
// The absmax is a block reduction; codes come from the magic-number quantizer
// with an exact fallback near ties (quant8_store), eight per store.
constexpr int kLdsRowF = 68;                 // 64 floats + 4 pad
constexpr int kLdsAF = 16 * kLdsRowF;        // one a (1024 b) = 16 padded rows
constexpr int kLdsFloats12288 = 6 * kLdsAF;

__device__ __forceinline__ float h2f_lo(uint32_t w) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xFFFFu)));
}
__device__ __forceinline__ float h2f_hi(uint32_t w) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16)));
}

// Eight magic-number results (nibble in bits 16..19) -> one dword of codes.
__device__ __forceinline__ uint32_t pack8_magic(const uint32_t* f) {
    // byte 2 of every result, even elements into `ev`, odd ones into `od`
    const uint32_t ev = __builtin_amdgcn_perm(__builtin_amdgcn_perm(f[6], f[4], 0x0c0c0602u),
                                              __builtin_amdgcn_perm(f[2], f[0], 0x0c0c0602u),
                                              0x05040100u);
    const uint32_t od = __builtin_amdgcn_perm(__builtin_amdgcn_perm(f[7], f[5], 0x0c0c0602u),
                                              __builtin_amdgcn_perm(f[3], f[1], 0x0c0c0602u),
                                              0x05040100u);
    return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
}

// True when any of eight magic-number results is within one unit of a tie.
__device__ __forceinline__ bool any_near_tie(const uint32_t* f) {
    const uint32_t m01 = min(f[0] & 0xFFFFu, f[1] & 0xFFFFu), m23 = min(f[2] & 0xFFFFu, f[3] & 0xFFFFu);
    const uint32_t m45 = min(f[4] & 0xFFFFu, f[5] & 0xFFFFu), m67 = min(f[6] & 0xFFFFu, f[7] & 0xFFFFu);
    return min(min(m01, m23), min(m45, m67)) < 3u;
}

// Codes of eight values z[k] whose true value is y_k = (z[k] * sg[k]) * norm,
// stored at element e (a multiple of 8) of an output row: one dword of
// nibbles (BITS = 4) or two dwords of bytes (BITS = 8).  The fast path (a
// normal, moderate scale s) uses the magic-number estimate with the constant
// c[k] = sg[k] * norm / s and falls back to the exact quotient near a tie.
template <int BITS>
__device__ __forceinline__ void quant8_store(uint8_t* row_out, int e, const float* z, const float* sg,
                                             const float* c, float norm, float s, bool fast) {
    if (BITS == 4) {
        uint32_t word = 0;
        bool exact = !fast;
        if (fast) {
            uint32_t f[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) f[k] = __float_as_uint(__builtin_fmaf(z[k], c[k], kQuantMagic));
            word = pack8_magic(f);
            exact = any_near_tie(f);
        }
        if (exact) {
            int c8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) c8[k] = quant_exact((z[k] * sg[k]) * norm, s);
            word = pack8(c8);
        }
        *reinterpret_cast<uint32_t*>(row_out + e / 2) = word;
    } else {
        uint32_t w0 = 0, w1 = 0;
        bool exact = !fast;
        if (fast) {
            uint32_t f[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) f[k] = __float_as_uint(__builtin_fmaf(z[k], c[k], kQuant8Magic));
            w0 = pack4_magic8(f);
            w1 = pack4_magic8(f + 4);
            exact = any_near_tie8(f);
        }
        if (exact) {
            int c8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) c8[k] = quant_exact8((z[k] * sg[k]) * norm, s);
            w0 = pack4b(c8);
            w1 = pack4b(c8 + 4);
        }
        *reinterpret_cast<uint2*>(row_out + e) = make_uint2(w0, w1);
    }
}

// One row per workgroup.  `one` is 1.0f passed at run time so that
// (x0 * one + x1) stays a mixed-precision FMA reading both fp16 halves.
template <int BITS, bool WRITE_ROT>
__global__ __launch_bounds__(256) void fwht_quant_k12288(
    const __half* __restrict__ X, float norm, float one, uint8_t* __restrict__ Xq,
    float* __restrict__ x_scale, float* __restrict__ X_rot) {
    __shared__ __attribute__((aligned(16))) float lds[kLdsFloats12288];
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const size_t row = blockIdx.x;

    // ---- phase 1: load x[a][4 beta .. 4 beta + 3], beta bits 0-3 permuted for DPP
    const int beta_in = g_perm(l16) | ((lane >> 4) << 4) | (wave << 6);
    uint2 raw[12];
    {
        const __half* xr = X + row * 12288 + 4 * beta_in;
#pragma unroll
        for (int a = 0; a < 12; ++a) {  // read once: non-temporal
            typedef unsigned int v2u __attribute__((ext_vector_type(2)));
            const v2u t = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(xr + a * 1024));
            raw[a] = make_uint2(t.x, t.y);
        }
    }
    const float s1 = lane_sign(l16, 0b0101), s2 = lane_sign(l16, 0b0110);
    const float s3 = lane_sign(l16, 0b1100), s4 = lane_sign(l16, 0b1000);

    // b bits 0-1 in registers; the first level reads both fp16 halves directly
    float v[12][4];
#pragma unroll
    for (int a = 0; a < 12; ++a) {
        const uint32_t w0 = raw[a].x, w1 = raw[a].y;
        const float s01 = __builtin_fmaf(h2f_lo(w0), one, h2f_hi(w0));
        const float d01 = __builtin_fmaf(h2f_hi(w0), -one, h2f_lo(w0));
        const float s23 = __builtin_fmaf(h2f_lo(w1), one, h2f_hi(w1));
        const float d23 = __builtin_fmaf(h2f_hi(w1), -one, h2f_lo(w1));
        v[a][0] = s01 + s23;
        v[a][1] = d01 + d23;
        v[a][2] = s01 - s23;
        v[a][3] = d01 - d23;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float col[12];
#pragma unroll
        for (int a = 0; a < 12; ++a) col[a] = v[a][j];
        h12_row(col);
#pragma unroll
        for (int a = 0; a < 12; ++a) v[a][j] = col[a];
    }
    dpp_wht16<48>(&v[0][0], s1, s2, s3, s4);

    const int ch = wave >> 1;
    const int blo = 8 * (((lane >> 4) & 3) | ((wave & 1) << 2));      // b & 63
    float z[6][8];
    const int beta = l16 | ((lane >> 4) << 4) | (wave << 6);
    float* dst = lds + (beta >> 4) * kLdsRowF + 4 * l16;
    const float* src = lds + g_perm(l16) * kLdsRowF + blo;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (half) __syncthreads();
#pragma unroll
        for (int c = 0; c < 6; ++c)
            *reinterpret_cast<float4*>(dst + c * kLdsAF) = make_float4(v[6*half+c][0], v[6*half+c][1], v[6*half+c][2], v[6*half+c][3]);
        __syncthreads();
        if (ch == half) {
#pragma unroll
            for (int ci = 0; ci < 6; ++ci) {
                const float4 p = *reinterpret_cast<const float4*>(src + ci * kLdsAF);
                const float4 q = *reinterpret_cast<const float4*>(src + ci * kLdsAF + 4);
                z[ci][0] = p.x; z[ci][1] = p.y; z[ci][2] = p.z; z[ci][3] = p.w;
                z[ci][4] = q.x; z[ci][5] = q.y; z[ci][6] = q.z; z[ci][7] = q.w;
            }
        }
    }
    dpp_wht16<48>(&z[0][0], s1, s2, s3, s4);

    // ---- absmax of the row
    float mx = 0.0f;
#pragma unroll
    for (int ci = 0; ci < 6; ++ci)
#pragma unroll
        for (int k = 0; k < 8; ++k) mx = __builtin_fmaxf(mx, __builtin_fabsf(z[ci][k]));
    const float amax = block_max_256(mx, red) * norm;   // = max_i fl32(|z_i| * norm)
    const float s = __fdiv_rn(amax, BITS == 4 ? kSeven : kQmax8);
    if (tid == 0) x_scale[row] = s;

    // Sign of each held value relative to the true transform: phase 1 left
    // (-1)^popcount(b2..b4), phase 2 (-1)^popcount(b6..b8); b2 is register bit 2.
    const int b3 = (lane >> 4) & 1, b4 = (lane >> 5) & 1;
    const bool neg_lo = ((b3 ^ b4) ^ (__builtin_popcount(l16 & 7) & 1)) != 0;
    const float sg_lo = neg_lo ? -1.0f : 1.0f;        // registers k = 0..3 (b2 = 0)
    const float sg_hi = -sg_lo;                        // registers k = 4..7 (b2 = 1)

    uint8_t* out = Xq + row * (BITS == 4 ? 6144 : 12288);
    const bool fast = (s >= 0x1p-100f) && (s <= 0x1p+100f);
    const float cr = fast ? norm * __fdiv_rn(1.0f, s) : 0.0f;
    float sg[8], c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        sg[k] = k < 4 ? sg_lo : sg_hi;
        c[k] = sg[k] * cr;
    }
#pragma unroll
    for (int ci = 0; ci < 6; ++ci)
        quant8_store<BITS>(out, (ch * 6 + ci) * 1024 + l16 * 64 + blo, z[ci], sg, c, norm, s, fast);
    if (WRITE_ROT) {
        float* yr = X_rot + row * 12288 + (ch * 6) * 1024 + l16 * 64 + blo;
#pragma unroll
        for (int ci = 0; ci < 6; ++ci) {
            float y[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = (z[ci][k] * (k < 4 ? sg_lo : sg_hi)) * norm;
            *reinterpret_cast<float4*>(yr + ci * 1024) = make_float4(y[0], y[1], y[2], y[3]);
            *reinterpret_cast<float4*>(yr + ci * 1024 + 4) = make_float4(y[4], y[5], y[6], y[7]);
        }
    }
}

// ---------------------------------------------------------------------------
// quant_rows: had_n = 1 (the rows are already in the rotated basis, e.g. R1
// folded upstream): per-token quantization only.  One workgroup of 256
// threads per row; thread t holds the chunks of 8 consecutive values t,
// t + 256, ... (NCH of them, one 16-byte fp16 load each), so the row never
// leaves registers: block absmax, then the magic-number quantizer with its
// exact fallback near ties, one store of codes per chunk.
template <typename TIn>
__device__ __forceinline__ void load_chunk8(const TIn* p, float* v);
template <>
__device__ __forceinline__ void load_chunk8<__half>(const __half* p, float* v) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    v[0] = h2f_lo(raw.x); v[1] = h2f_hi(raw.x); v[2] = h2f_lo(raw.y); v[3] = h2f_hi(raw.y);
    v[4] = h2f_lo(raw.z); v[5] = h2f_hi(raw.z); v[6] = h2f_lo(raw.w); v[7] = h2f_hi(raw.w);
}
template <>
__device__ __forceinline__ void load_chunk8<float>(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <int BITS, typename TIn, int NCH, bool WRITE_ROT>
__global__ __launch_bounds__(256) void quant_rows(const TIn* __restrict__ X, int K,
                                                  uint8_t* __restrict__ Xq,
                                                  float* __restrict__ x_scale,
                                                  float* __restrict__ X_rot) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const size_t row = blockIdx.x;
    const int nch = K / 8;
    float v[NCH][8];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = tid + 256 * i;
        if (c < nch) {
            load_chunk8<TIn>(X + row * K + 8 * c, v[i]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[i][k] = 0.0f;
        }
    }
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[i][k]));
    const float s = __fdiv_rn(block_max_256(mx, red), BITS == 4 ? kSeven : kQmax8);
    if (tid == 0) x_scale[row] = s;
    uint8_t* out = Xq + row * static_cast<size_t>(BITS == 4 ? K / 2 : K);
    const bool fast = (s >= 0x1p-100f) && (s <= 0x1p+100f);
    const float cr = fast ? __fdiv_rn(1.0f, s) : 0.0f;
    const float one[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
    const float crs[8] = {cr, cr, cr, cr, cr, cr, cr, cr};
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = tid + 256 * i;
        if (c >= nch) break;
        quant8_store<BITS>(out, 8 * c, v[i], one, crs, 1.0f, s, fast);
        if (WRITE_ROT) {
            float4* yr = reinterpret_cast<float4*>(X_rot + row * K + 8 * c);
            yr[0] = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
            yr[1] = make_float4(v[i][4], v[i][5], v[i][6], v[i][7]);
        }
    }
}

template <int BITS, typename TIn, bool WR>
hipError_t launch_quant_rows(const TIn* X, int M, int K, uint8_t* Xq, float* xs, float* Xr,
                             hipStream_t s) {
    const int nch = K / 8;
    if (nch <= 256)
        hipLaunchKernelGGL((quant_rows<BITS, TIn, 1, WR>), dim3(M), dim3(256), 0, s, X, K, Xq, xs, Xr);
    else if (nch <= 512)
        hipLaunchKernelGGL((quant_rows<BITS, TIn, 2, WR>), dim3(M), dim3(256), 0, s, X, K, Xq, xs, Xr);
    else if (nch <= 1024)
        hipLaunchKernelGGL((quant_rows<BITS, TIn, 4, WR>), dim3(M), dim3(256), 0, s, X, K, Xq, xs, Xr);
    else
        hipLaunchKernelGGL((quant_rows<BITS, TIn, 8, WR>), dim3(M), dim3(256), 0, s, X, K, Xq, xs, Xr);
    return hipGetLastError();
}

template <int BITS, typename TIn, bool WR>
hipError_t launch_rowlds(const TIn* X, int M, int K, HadOrder h, uint8_t* Xq, float* xs,
                         float* Xr, hipStream_t s) {
    const size_t lds = static_cast<size_t>(K) * sizeof(float);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&fwht_quant_rowlds<BITS, TIn, WR>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 64);
    if (attr != hipSuccess) return attr;
    const float norm = (h.n > 1) ? static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(h.n))) : 1.0f;
    hipLaunchKernelGGL((fwht_quant_rowlds<BITS, TIn, WR>), dim3(M), dim3(kRowThreads), lds, s, X, K,
                       h.log2p, h.has12 ? 1 : 0, h.n > 1 ? 1 : 0, norm, Xq, xs, Xr);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_fwht_quant_bits(const void* X, bool x_f16, int M, int K, HadOrder h, uint8_t* Xq,
                                  float* x_scale, float* X_rot, hipStream_t s) {
    if (x_f16 && h.n == 12288 && K == 12288) {
        const float norm = static_cast<float>(1.0 / __builtin_sqrt(12288.0));
        const __half* x = static_cast<const __half*>(X);
        if (X_rot)
            hipLaunchKernelGGL((fwht_quant_k12288<BITS, true>), dim3(M), dim3(256), 0, s, x, norm, 1.0f, Xq,
                               x_scale, X_rot);
        else
            hipLaunchKernelGGL((fwht_quant_k12288<BITS, false>), dim3(M), dim3(256), 0, s, x, norm, 1.0f, Xq,
                               x_scale, X_rot);
        return hipGetLastError();
    }
    if (h.n == 1 && K <= 16384) {
        if (x_f16) {
            const __half* x = static_cast<const __half*>(X);
            return X_rot ? launch_quant_rows<BITS, __half, true>(x, M, K, Xq, x_scale, X_rot, s)
                         : launch_quant_rows<BITS, __half, false>(x, M, K, Xq, x_scale, X_rot, s);
        }
        const float* x = static_cast<const float*>(X);
        return X_rot ? launch_quant_rows<BITS, float, true>(x, M, K, Xq, x_scale, X_rot, s)
                     : launch_quant_rows<BITS, float, false>(x, M, K, Xq, x_scale, X_rot, s);
    }
    if (x_f16) {
        const __half* x = static_cast<const __half*>(X);
        return X_rot ? launch_rowlds<BITS, __half, true>(x, M, K, h, Xq, x_scale, X_rot, s)
                     : launch_rowlds<BITS, __half, false>(x, M, K, h, Xq, x_scale, X_rot, s);
    }
    const float* x = static_cast<const float*>(X);
    return X_rot ? launch_rowlds<BITS, float, true>(x, M, K, h, Xq, x_scale, X_rot, s)
                 : launch_rowlds<BITS, float, false>(x, M, K, h, Xq, x_scale, X_rot, s);
}

}  // namespace

hipError_t launch_fwht_quant(const void* X, bool x_f16, int M, int K, HadOrder h, int bits, uint8_t* Xq,
                             float* x_scale, float* X_rot, hipStream_t s) {
    return bits == 8 ? launch_fwht_quant_bits<8>(X, x_f16, M, K, h, Xq, x_scale, X_rot, s)
                     : launch_fwht_quant_bits<4>(X, x_f16, M, K, h, Xq, x_scale, X_rot, s);
}

}  // namespace spin
