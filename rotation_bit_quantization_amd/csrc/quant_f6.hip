// spin_fwht_quant_f6 with had_n = 1: activations already in the rotated basis
// (R1 or R2 folded into the weights, page "SpinQuant, Reproduced", Q5) are
// only quantized per token to INT4 (abstract: 4-bit activations), and the
// codes go straight into the FP6 operand layout of include/libspin.h with each
// row's code sum, so spin_w4a4_gemm_f6f6 can take them without a separate
// spin_codes_f6 pass.
//
// One workgroup of 256 threads per row, as quant_rows (rows placed per XCD, see
// quant_rows_f6): thread t holds the
// 16-code chunks t, t + 256, ... (two 16-byte fp16 loads, or four fp32 ones,
// each), the block absmax gives s = fl32(absmax / 7), and every code is formed
// exactly as quant_rows forms it (the magic-number estimate, the exact IEEE
// quotient near a tie or outside the fast range), so the codes and scales are
// the bits spin_fwht_quant(X, had_n = 1) writes.  A chunk's sixteen codes
// become one 12-byte field group (spread16_offset, the encoding the tiles and
// spin_codes_f6 use) stored at its place in the layout; the code sums come
// from v_dot8_i32_i4 on the packed nibbles and one block reduction.
#include "fwht12288.h"
#include "libspin.h"
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

template <typename TIn>
__device__ __forceinline__ void load16(const TIn* p, float* v);
template <>
__device__ __forceinline__ void load16<__half>(const __half* p, float* v) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint4 b = *reinterpret_cast<const uint4*>(p + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = h2f_lo(w[i]);
        v[2 * i + 1] = h2f_hi(w[i]);
    }
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 a = reinterpret_cast<const float4*>(p)[i];
        v[4 * i] = a.x;
        v[4 * i + 1] = a.y;
        v[4 * i + 2] = a.z;
        v[4 * i + 3] = a.w;
    }
}

// Eight codes of y = z (no rotation) as one dword of nibbles: the arithmetic of
// quant8_store<4> with unit signs and norm.
__device__ __forceinline__ uint32_t codes8(const float* z, float cr, float s, bool fast) {
    if (fast) {
        uint32_t f[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = __float_as_uint(__builtin_fmaf(z[k], cr, kQuantMagic));
        if (!any_near_tie(f)) return pack8_magic(f);
    }
    int c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = quant_exact(z[k], s);
    return pack8(c);
}

// Rows map to workgroups so that each XCD (workgroups b with the same b % 8)
// owns whole 32-row blocks: the 24-byte pieces of a 1536-byte region, one per
// row, then all pass through one L2 (interleaved over the XCDs, the partial
// lines of a region are written back from eight of them).
template <typename TIn, int NCH>
__global__ __launch_bounds__(256) void quant_rows_f6(const TIn* __restrict__ X, int M, int K, int rows_per_xcd,
                                                     uint8_t* __restrict__ Xf6, int32_t* __restrict__ x_sum,
                                                     float* __restrict__ x_scale) {
    __shared__ float red[4];
    __shared__ int sums[4];
    const int tid = threadIdx.x;
    const int r = static_cast<int>(blockIdx.x % 8) * rows_per_xcd + static_cast<int>(blockIdx.x / 8);
    if (r >= M) return;   // the whole workgroup
    const size_t row = static_cast<size_t>(r);
    const int nch = K / 16;
    float v[NCH][16];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = tid + 256 * i;
        if (c < nch) {
            load16<TIn>(X + row * K + 16 * c, v[i]);
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) v[i][k] = 0.0f;
        }
    }
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int k = 0; k < 16; ++k) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[i][k]));
    const float s = __fdiv_rn(block_max_256(mx, red), kSeven);
    if (tid == 0) x_scale[row] = s;
    const bool fast = (s >= 0x1p-100f) && (s <= 0x1p+100f);
    const float cr = fast ? __fdiv_rn(1.0f, s) : 0.0f;
    // region (row / 32, k / 64), k-half (k / 32) % 2, this row, 16-code group (k / 16) % 2
    uint8_t* base = Xf6 + (row >> 5) * static_cast<size_t>(K / 64) * 1536 + (row & 31) * 24;
    int sum = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = tid + 256 * i;
        if (c >= nch) break;
        const uint32_t w0 = codes8(v[i], cr, s, fast), w1 = codes8(v[i] + 8, cr, s, fast);
        sum = __builtin_amdgcn_sdot8(static_cast<int>(w0), 0x11111111, sum, false);
        sum = __builtin_amdgcn_sdot8(static_cast<int>(w1), 0x11111111, sum, false);
        uint32_t o[3];
        spread16_offset(w0, w1, o);
        const int e = 16 * c;
        *reinterpret_cast<uint3*>(base + (e >> 6) * 1536 + ((e >> 5) & 1) * 768 + ((e >> 4) & 1) * 12) =
            make_uint3(o[0], o[1], o[2]);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m, 64);
    if ((tid & 63) == 0) sums[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0) x_sum[row] = sums[0] + sums[1] + sums[2] + sums[3];
}

template <typename TIn>
hipError_t launch_t(const TIn* X, int M, int K, uint8_t* Xf6, int32_t* x_sum, float* x_scale, hipStream_t s) {
    const int nch = K / 16;
    const int rows_per_xcd = (M + 8 * 32 - 1) / (8 * 32) * 32;
    const dim3 grid(static_cast<unsigned>(8 * rows_per_xcd));
    if (nch <= 256)
        hipLaunchKernelGGL((quant_rows_f6<TIn, 1>), grid, dim3(256), 0, s, X, M, K, rows_per_xcd, Xf6, x_sum, x_scale);
    else if (nch <= 512)
        hipLaunchKernelGGL((quant_rows_f6<TIn, 2>), grid, dim3(256), 0, s, X, M, K, rows_per_xcd, Xf6, x_sum, x_scale);
    else
        hipLaunchKernelGGL((quant_rows_f6<TIn, 4>), grid, dim3(256), 0, s, X, M, K, rows_per_xcd, Xf6, x_sum, x_scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows_f6(const void* X, bool x_f16, int M, int K, uint8_t* Xf6, int32_t* x_sum,
                                float* x_scale, hipStream_t s) {
    if (K % 128 != 0 || K > SPIN_FWHT_F6_QUANT_MAX_K) return hipErrorInvalidValue;
    return x_f16 ? launch_t(static_cast<const __half*>(X), M, K, Xf6, x_sum, x_scale, s)
                 : launch_t(static_cast<const float*>(X), M, K, Xf6, x_sum, x_scale, s);
}

}  // namespace spin
