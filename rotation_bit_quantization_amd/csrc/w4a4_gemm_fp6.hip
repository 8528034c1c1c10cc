// spin_w4a4_gemm on the gfx950 FP6 matrix cores: one workgroup per 256 x 256
// output tile (the tile body, its encoding and its measurements are in
// gemm_fp6_tile.h), and the choice between this kernel and the int8 ones.
#include "gemm_fp6_tile.h"
#include "libspin.h"
#include "spin_internal.h"

namespace spin {
namespace {

using namespace fp6;

template <bool WRITE_ACC>
__global__ __launch_bounds__(kF6Threads) void w4a4_gemm_fp6(
    const uint8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * kF6StageBytes];
    int tm, tn;
    tile_of(blockIdx.x, (M + kF6T - 1) / kF6T, (N + kF6T - 1) / kF6T, &tm, &tn);
    gemm_tile<WRITE_ACC>(Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out, tm, tn, lds);
}

template <bool WRITE_ACC>
__global__ __launch_bounds__(kF6Threads) void w4a4_gemm_fp6_f6a(
    const uint8_t* __restrict__ Xf6, const int32_t* __restrict__ x_sum, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * kF6StageBytes];
    int tm, tn;
    tile_of(blockIdx.x, (M + kF6T - 1) / kF6T, (N + kF6T - 1) / kF6T, &tm, &tn);
    gemm_tile_f6a<WRITE_ACC>(Xf6, x_sum, x_scale, Wq, w_scale, M, N, K, Y, acc_out, tm, tn, lds);
}

}  // namespace

// Measured on MI355X against the int8 kernels (random codes, µs):
//   M x N x K             FP6     int8
//   4096 x 4096 x 12288   172.9   198.5
//   8192 x 4096 x 12288   367.8   373.6
//   4096 x 4096 x 8192    122.9   131.9
//   16384 x 4096 x 12288  725.0   703.7
//   2048 x 4096 x 12288   153.9   146.9   (128 tiles: half the CUs)
//   256 x 4096 x 12288    140.5   128.8
//   4096 x 6144 x 4096    143.5   122.3   (K = 4096: int8, 256 x 384 tiles)
// The FP6 kernel wins on long reductions whose 256 x 256 tiles fill one or
// two rounds of the compute units; with fewer tiles the int8 kernels' shorter
// per-tile latency wins, with many rounds their higher sustained rate.
// Up to 64 rows, and up to 128 when N / 16 < 4 CUs, the weight-streaming
// decode kernel takes the product.
bool w4a4_gemm_fp6_applies(int M, int N, int K) {
    if (M <= 64 || K % kF6StepCodes != 0 || K < 8192 || K > kGemmFp6MaxK) return false;
    const int cus = device_cu_count();
    if (cus <= 0) return false;
    if (M <= 128 && (N + 15) / 16 < 4 * cus) return false;   // the weight-streaming kernel's range
    const long long tiles = static_cast<long long>((M + kF6T - 1) / kF6T) * ((N + kF6T - 1) / kF6T);
    return 4 * tiles >= 3LL * cus && tiles <= 2LL * cus;
}

hipError_t launch_w4a4_gemm_fp6(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                                const float* w_scale, int M, int N, int K, float* Y,
                                int32_t* acc_out, hipStream_t s) {
    // the pipeline converts two steps before the first multiplication
    static_assert(SPIN_GEMM_FP6_MIN_K == 2 * kF6StepCodes && SPIN_GEMM_FP6_MAX_K == kGemmFp6MaxK,
                  "the FP6 K range of the ABI");
    if (K % kF6StepCodes != 0 || K < 2 * kF6StepCodes || K > kGemmFp6MaxK) return hipErrorInvalidValue;
    const long long tiles = static_cast<long long>((M + kF6T - 1) / kF6T) * ((N + kF6T - 1) / kF6T);
    const dim3 grid(static_cast<unsigned>(tiles));
    if (acc_out)
        hipLaunchKernelGGL((w4a4_gemm_fp6<true>), grid, dim3(kF6Threads), 0, s, Xq, x_scale, Wq, w_scale, M, N,
                           K, Y, acc_out);
    else
        hipLaunchKernelGGL((w4a4_gemm_fp6<false>), grid, dim3(kF6Threads), 0, s, Xq, x_scale, Wq, w_scale, M,
                           N, K, Y, acc_out);
    return hipGetLastError();
}

hipError_t launch_w4a4_gemm_f6(const uint8_t* Xf6, const int32_t* x_sum, const float* x_scale, const uint8_t* Wq,
                               const float* w_scale, int M, int N, int K, float* Y, int32_t* acc_out,
                               hipStream_t s) {
    if (K % kF6StepCodes != 0 || K < 2 * kF6StepCodes || K > kGemmFp6MaxK) return hipErrorInvalidValue;
    const long long tiles = static_cast<long long>((M + kF6T - 1) / kF6T) * ((N + kF6T - 1) / kF6T);
    const dim3 grid(static_cast<unsigned>(tiles));
    if (acc_out)
        hipLaunchKernelGGL((w4a4_gemm_fp6_f6a<true>), grid, dim3(kF6Threads), 0, s, Xf6, x_sum, x_scale, Wq,
                           w_scale, M, N, K, Y, acc_out);
    else
        hipLaunchKernelGGL((w4a4_gemm_fp6_f6a<false>), grid, dim3(kF6Threads), 0, s, Xf6, x_sum, x_scale, Wq,
                           w_scale, M, N, K, Y, acc_out);
    return hipGetLastError();
}

}  // namespace spin
