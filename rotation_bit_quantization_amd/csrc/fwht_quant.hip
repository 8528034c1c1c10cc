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
//
// fwht_quant_k12288_mfma: fp16 rows of 12288 with had_n = 12288 (the R4 /
// down_proj case), one wave per row, the two 32-point stages of each
// 1024-block on the matrix cores and the order-12 mix in registers (see the
// kernel).  fwht_quant_k12288_wg: the same arithmetic with four waves per
// row, for batches of up to kWgMaxRows rows (decode), bit-identical.
#include "fwht12288.h"
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
// The FP6-layout producer: one wave (workgroup of 64) per row, rows mapped to
// workgroups so that each XCD (workgroups b with the same b % 8) owns whole
// 32-row blocks: the rows of a 1536-byte region are written through one L2.
__global__ __launch_bounds__(64, 2) void fwht_quant_k12288_f6(const __half* __restrict__ X, float norm, float mone,
                                                              int M, int rows_per_xcd, uint8_t* __restrict__ Xf6,
                                                              int32_t* __restrict__ x_sum,
                                                              float* __restrict__ x_scale) {
    const int row = static_cast<int>(blockIdx.x % 8) * rows_per_xcd + static_cast<int>(blockIdx.x / 8);
    if (row >= M) return;
    fwht12288_row_f6(X, static_cast<size_t>(row), threadIdx.x, norm, mone, Xf6, x_sum, x_scale);
}

// One wave (workgroup of 64) per row.
template <int BITS, bool WRITE_ROT>
__global__ __launch_bounds__(64, 2) void fwht_quant_k12288_mfma(
    const __half* __restrict__ X, float norm, float mone, uint8_t* __restrict__ Xq,
    float* __restrict__ x_scale, float* __restrict__ X_rot) {
    fwht12288_row<BITS, WRITE_ROT>(X, blockIdx.x, threadIdx.x, norm, mone, Xq, x_scale, X_rot);
}

// ---------------------------------------------------------------------------
// fwht_quant_k12288_wg: the same transform for a few rows (decode batches),
// where one wave per row leaves most of the chip idle and a row's latency is
// the kernel's time.  Four waves share a row: wave w runs the two matrix-core
// stages of blocks 3w .. 3w + 2 exactly as fwht_quant_k12288_mfma does, the
// stage-2 results go through 48 KB of LDS, and each thread then takes four
// consecutive elements of every block (element e0 .. e0 + 3 of the block, the
// registers r0 .. r0 + 3 of stage lane L) for the H12 mix, the absmax and the
// quantizer.  Every value goes through the same operations as in the one-wave
// kernel, so the two produce the same bits.

// Four consecutive codes (2 bytes of nibbles, or 4 bytes) from the
// magic-number quantizer, exact quotient near a tie or outside the fast range.
template <int BITS>
__device__ __forceinline__ void quant4_store(uint8_t* p, const float (&u)[4], float cr, float nrm, float s,
                                             bool fast) {
    uint32_t w = 0;
    bool exact = !fast;
    if (fast) {
        uint32_t f[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            f[k] = __float_as_uint(__builtin_fmaf(u[k], cr, BITS == 4 ? kQuantMagic : kQuant8Magic));
        if (BITS == 4) {
            w = ((f[0] >> 16) & 0xFu) | ((f[1] >> 12) & 0xF0u) | ((f[2] >> 8) & 0xF00u) | ((f[3] >> 4) & 0xF000u);
            exact = (static_cast<int>(near_tie(f[0])) | static_cast<int>(near_tie(f[1])) |
                     static_cast<int>(near_tie(f[2])) | static_cast<int>(near_tie(f[3]))) != 0;
        } else {
            w = pack4_magic8(f);
            exact = (static_cast<int>(near_tie8(f[0])) | static_cast<int>(near_tie8(f[1])) |
                     static_cast<int>(near_tie8(f[2])) | static_cast<int>(near_tie8(f[3]))) != 0;
        }
    }
    if (exact) {
        int c[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = BITS == 4 ? quant_exact(u[k] * nrm, s) : quant_exact8(u[k] * nrm, s);
        w = BITS == 4 ? ((c[0] & 15) | ((c[1] & 15) << 4) | ((c[2] & 15) << 8) | ((c[3] & 15) << 12)) : pack4b(c);
    }
    if (BITS == 4)
        *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(w);
    else
        *reinterpret_cast<uint32_t*>(p) = w;
}

constexpr int kWgRowThreads = 256;
// Up to this many rows the four-waves-per-row kernel is the faster one (measured:
// 5.6 against 8.7 us at 16 rows, 7.5 against 10.5 us at 512, 13.2 against
// 12.7 us at 1024).
constexpr int kWgMaxRows = 512;

template <int BITS, bool WRITE_ROT>
__global__ __launch_bounds__(kWgRowThreads) void fwht_quant_k12288_wg(
    const __half* __restrict__ X, float norm, float mone, uint8_t* __restrict__ Xq,
    float* __restrict__ x_scale, float* __restrict__ X_rot) {
    __shared__ __attribute__((aligned(16))) float ex[12 * 64 * 16];   // [block][stage lane][register]
    __shared__ float red[4];
    __shared__ uint32_t redb[4];
    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const size_t row = blockIdx.x;
    const __half* xr = X + row * 12288 + 32 * (lane & 31) + 16 * (lane >> 5);

    u4v raw[3][2];
#pragma unroll
    for (int j = 0; j < 3; ++j) {  // read once: non-temporal
        raw[j][0] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(xr + (3 * wave + j) * 1024));
        raw[j][1] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(xr + (3 * wave + j) * 1024 + 8));
    }
    u4v sa, sb;
    operand_signs(lane, sa, sb);

    // this thread's elements after the exchange
    const int L = (t >> 1) & 63, r0 = 8 * (t >> 7) + 4 * (t & 1);
    float nrm = norm * 32.0f;
    unsigned magpair = 0x28002800u;     // +-2^-5
    float y[12][4];
    float amax = 0.0f;
    for (int pass = 0; pass < 2; ++pass) {
        const h8v b1a = __builtin_bit_cast(h8v, sa | magpair), b1b = __builtin_bit_cast(h8v, sb | magpair);
        const h8v b2a = __builtin_bit_cast(h8v, sa | 0x3C003C00u), b2b = __builtin_bit_cast(h8v, sb | 0x3C003C00u);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const f16v u = hadamard1024_mfma(raw[j][0], raw[j][1], b1a, b1b, b2a, b2b, mone);
            float4* dst = reinterpret_cast<float4*>(ex + ((3 * wave + j) * 64 + lane) * 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = make_float4(u[4 * q], u[4 * q + 1], u[4 * q + 2], u[4 * q + 3]);
        }
        __syncthreads();
#pragma unroll
        for (int a = 0; a < 12; ++a) {
            const float4 v = *reinterpret_cast<const float4*>(ex + (a * 64 + L) * 16 + r0);
            y[a][0] = v.x; y[a][1] = v.y; y[a][2] = v.z; y[a][3] = v.w;
        }
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float col12[12];
#pragma unroll
            for (int a = 0; a < 12; ++a) col12[a] = y[a][i];
            h12_row(col12);
#pragma unroll
            for (int a = 0; a < 12; ++a) {
                y[a][i] = col12[a];
                mx = __builtin_fmaxf(mx, __builtin_fabsf(col12[a]));
            }
        }
        amax = block_max_256(mx, red) * nrm;       // = max_i fl32(|u_i| * nrm); ends with a barrier
        if (amax >= 2.0f || pass == 1) break;
        // small (or all-zero) row: rescale stage 1 from the exact largest |x|
        uint32_t mb = 0;
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                mb = max(mb, max(raw[j][0][k] & 0x7FFFu, (raw[j][0][k] >> 16) & 0x7FFFu));
                mb = max(mb, max(raw[j][1][k] & 0x7FFFu, (raw[j][1][k] >> 16) & 0x7FFFu));
            }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) mb = max(mb, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mb), o, 64)));
        if (lane == 0) redb[wave] = mb;
        __syncthreads();
        mb = max(max(redb[0], redb[1]), max(redb[2], redb[3]));
        const int m = min(20, 29 - static_cast<int>(mb >> 10));   // m >= -2 for any fp16 row
        nrm = __builtin_ldexpf(norm, 5 - m);
        magpair = __builtin_bit_cast(unsigned short, static_cast<_Float16>(__builtin_ldexpf(1.0f, m - 5))) * 0x10001u;
    }

    const float s = __fdiv_rn(amax, BITS == 4 ? kSeven : kQmax8);
    if (t == 0) x_scale[row] = s;
    const bool fast = (s >= 0x1p-100f) && (s <= 0x1p+100f);
    const float cr = fast ? nrm * __fdiv_rn(1.0f, s) : 0.0f;
    const unsigned e0 = 32u * (L & 31) + 16u * (L >> 5) + r0;
    uint8_t* out = Xq + row * (BITS == 4 ? 6144 : 12288) + e0 * BITS / 8;
#pragma unroll
    for (int a = 0; a < 12; ++a) quant4_store<BITS>(out + a * (1024 * BITS / 8), y[a], cr, nrm, s, fast);
    if (WRITE_ROT) {
        float* yr = X_rot + row * 12288 + e0;
#pragma unroll
        for (int a = 0; a < 12; ++a)
            *reinterpret_cast<float4*>(yr + a * 1024) =
                make_float4(y[a][0] * nrm, y[a][1] * nrm, y[a][2] * nrm, y[a][3] * nrm);
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
        if (M <= kWgMaxRows) {
            if (X_rot)
                hipLaunchKernelGGL((fwht_quant_k12288_wg<BITS, true>), dim3(M), dim3(kWgRowThreads), 0, s, x, norm,
                                   -1.0f, Xq, x_scale, X_rot);
            else
                hipLaunchKernelGGL((fwht_quant_k12288_wg<BITS, false>), dim3(M), dim3(kWgRowThreads), 0, s, x, norm,
                                   -1.0f, Xq, x_scale, X_rot);
            return hipGetLastError();
        }
        if (X_rot)
            hipLaunchKernelGGL((fwht_quant_k12288_mfma<BITS, true>), dim3(M), dim3(64), 0, s, x, norm, -1.0f, Xq,
                               x_scale, X_rot);
        else
            hipLaunchKernelGGL((fwht_quant_k12288_mfma<BITS, false>), dim3(M), dim3(64), 0, s, x, norm, -1.0f, Xq,
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

hipError_t launch_fwht_quant_f6(const __half* X, int M, uint8_t* Xf6, int32_t* x_sum, float* x_scale,
                                hipStream_t s) {
    const int rows_per_xcd = (M + 8 * 32 - 1) / (8 * 32) * 32;
    const float norm = static_cast<float>(1.0 / __builtin_sqrt(12288.0));
    hipLaunchKernelGGL(fwht_quant_k12288_f6, dim3(static_cast<unsigned>(8 * rows_per_xcd)), dim3(64), 0, s, X, norm,
                       -1.0f, M, rows_per_xcd, Xf6, x_sum, x_scale);
    return hipGetLastError();
}

}  // namespace spin
