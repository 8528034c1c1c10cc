// spin_fwht_quant kernels: online Hadamard of each activation row followed by
// per-token symmetric INT4 (page "SpinQuant, Reproduced", Q5: R4 before
// down_proj runs online as a Hadamard over the MLP width; abstract: 4-bit
// activations).
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

template <typename TIn, bool WRITE_ROT>
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
    const float s = __fdiv_rn(amax, kSeven);
    if (tid == 0) x_scale[m] = s;

    uint32_t* out = reinterpret_cast<uint32_t*>(Xq + m * static_cast<size_t>(K / 2));
    for (int g = tid; g < K / 8; g += kRowThreads) {
        int c8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c8[j] = quant_exact(row[8 * g + j], s);
        out[g] = pack8(c8);
    }
    if (WRITE_ROT) {
        float* yr = X_rot + m * static_cast<size_t>(K);
        for (int i = tid; i < K; i += kRowThreads) yr[i] = row[i];
    }
}

template <typename TIn, bool WR>
hipError_t launch_rowlds(const TIn* X, int M, int K, HadOrder h, uint8_t* Xq, float* xs,
                         float* Xr, hipStream_t s) {
    const size_t lds = static_cast<size_t>(K) * sizeof(float);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&fwht_quant_rowlds<TIn, WR>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 64);
    if (attr != hipSuccess) return attr;
    const float norm = (h.n > 1) ? static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(h.n))) : 1.0f;
    hipLaunchKernelGGL((fwht_quant_rowlds<TIn, WR>), dim3(M), dim3(kRowThreads), lds, s, X, K,
                       h.log2p, h.has12 ? 1 : 0, h.n > 1 ? 1 : 0, norm, Xq, xs, Xr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwht_quant(const void* X, bool x_f16, int M, int K, HadOrder h, uint8_t* Xq,
                             float* x_scale, float* X_rot, hipStream_t s) {
    if (x_f16) {
        const __half* x = static_cast<const __half*>(X);
        return X_rot ? launch_rowlds<__half, true>(x, M, K, h, Xq, x_scale, X_rot, s)
                     : launch_rowlds<__half, false>(x, M, K, h, Xq, x_scale, X_rot, s);
    }
    const float* x = static_cast<const float*>(X);
    return X_rot ? launch_rowlds<float, true>(x, M, K, h, Xq, x_scale, X_rot, s)
                 : launch_rowlds<float, false>(x, M, K, h, Xq, x_scale, X_rot, s);
}

}  // namespace spin
