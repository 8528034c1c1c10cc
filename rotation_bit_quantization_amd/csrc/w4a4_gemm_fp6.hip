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

// Split-K: block b takes K slice `sl` of one tile.  Blocks are put in an
// order in which each XCD holds a contiguous range of (slice, tile) pairs,
// the tiles of one slice column-major (the few row blocks of a column share
// its weight tile in the XCD's L2).
__global__ __launch_bounds__(kF6Threads) void w4a4_gemm_fp6_split(
    const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Wq, int M, int N, int K, int slices,
    float* __restrict__ Y) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * kF6StageBytes];
    const int tiles_m = (M + kF6T - 1) / kF6T, tiles_n = (N + kF6T - 1) / kF6T;
    const int tiles = tiles_m * tiles_n;
    const int total = tiles * slices;
    int w = static_cast<int>(blockIdx.x);
    if ((total & 7) == 0) w = (w & 7) * (total >> 3) + (w >> 3);
    const int sl = w / tiles, t = w - sl * tiles;
    const int steps = K / kF6StepCodes;
    const int s0 = sl * steps / slices, s1 = (sl + 1) * steps / slices;
    gemm_tile<false, true>(Xq, nullptr, Wq, nullptr, M, N, K, Y, nullptr, t % tiles_m, t / tiles_m, lds, s0,
                           s1 - s0);
}

// Zeroes the int32 partial sums (a kernel rather than a memset, so that the
// three launches of a split product can be captured in a graph).
__global__ __launch_bounds__(256) void zero_partials(int32_t* __restrict__ p, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

// Row blockIdx.x of the summed int32 accumulators in Y -> the dequantized
// float32 outputs, in place, with the epilogue arithmetic of the tile.
template <bool WRITE_ACC>
__global__ __launch_bounds__(256) void split_dequant(float* __restrict__ Y, const float* __restrict__ x_scale,
                                                     const float* __restrict__ w_scale, int N,
                                                     int32_t* __restrict__ acc_out) {
    const int row = static_cast<int>(blockIdx.x);
    const float sx = x_scale[row];
    float* y = Y + static_cast<size_t>(row) * N;
    for (int col = static_cast<int>(blockIdx.y * blockDim.x + threadIdx.x); col < N;
         col += static_cast<int>(gridDim.y * blockDim.x)) {
        const int a = __builtin_bit_cast(int, y[col]);
        float v = static_cast<float>(a) * sx;
        v = v * w_scale[col];
        y[col] = v;
        if (WRITE_ACC) acc_out[static_cast<size_t>(row) * N + col] = a;
    }
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

// Number of K slices for the split-K form, 0 where it does not apply.  A
// slice costs about its steps of 128 codes plus two (the pipeline's fill and
// the epilogue) at kStepUs each, and its atomic additions kAtomicUs per
// million outputs (measured: 16.8 M no-return int32 atomic additions take
// about 41 us on MI355X, whatever the contention); the slice count that
// minimises the sum is taken, among powers of two that keep every slice at
// two steps or more and all slices in one round of the compute units.
// AUTO takes it only past the weight-streaming kernel's 128 rows, where the
// tiles leave at least half of the compute units idle, and when the model
// (with the fill and dequantizing passes priced at HBM speed) predicts a
// saving of a sixth or more over one round of whole tiles.
int w4a4_gemm_fp6_split_slices(int M, int N, int K, bool forced) {
    constexpr double kStepUs = 3500.0 / 2400.0;
    constexpr double kAtomicUs = 41.0 / 16.8;
    constexpr double kPassUsPerMillion = 12.0 / 5.0;   // 12 bytes per output at 5 TB/s
    if (M <= 0 || N <= 0 || K % kF6StepCodes != 0 || K < 2 * kF6StepCodes || K > kGemmFp6MaxK) return 0;
    const int cus = device_cu_count();
    if (cus <= 0) return 0;
    const long long tiles = static_cast<long long>((M + kF6T - 1) / kF6T) * ((N + kF6T - 1) / kF6T);
    if (!forced && (M <= 128 || 2 * tiles > cus)) return 0;
    const int steps = K / kF6StepCodes;
    const double outputs = static_cast<double>(M) * N / 1e6;
    auto cost = [&](int S) { return ((steps + S - 1) / S + 2) * kStepUs + S * outputs * kAtomicUs; };
    int best = 1;
    for (int S = 2; steps / S >= 2 && tiles * S <= cus; S *= 2)
        if (cost(S) < cost(best)) best = S;
    if (forced) return best;
    const double whole = ((tiles + cus - 1) / cus) * (steps + 2) * kStepUs;
    if (best < 2 || 6.0 * (cost(best) + outputs * kPassUsPerMillion) > 5.0 * whole) return 0;
    return best;
}

hipError_t launch_w4a4_gemm_fp6_split(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                                      const float* w_scale, int M, int N, int K, int slices, float* Y,
                                      int32_t* acc_out, hipStream_t s) {
    if (K % kF6StepCodes != 0 || K < 2 * kF6StepCodes || K > kGemmFp6MaxK || slices < 1 ||
        K / kF6StepCodes < 2 * slices)
        return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    const size_t n = static_cast<size_t>(M) * N;
    const unsigned zb = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 8192));
    hipLaunchKernelGGL(zero_partials, dim3(zb), dim3(256), 0, s, reinterpret_cast<int32_t*>(Y), n);
    const long long tiles = static_cast<long long>((M + kF6T - 1) / kF6T) * ((N + kF6T - 1) / kF6T);
    hipLaunchKernelGGL(w4a4_gemm_fp6_split, dim3(static_cast<unsigned>(tiles * slices)), dim3(kF6Threads), 0, s,
                       Xq, Wq, M, N, K, slices, Y);
    const dim3 fin(static_cast<unsigned>(M), static_cast<unsigned>((N + 1023) / 1024));
    if (acc_out)
        hipLaunchKernelGGL((split_dequant<true>), fin, dim3(256), 0, s, Y, x_scale, w_scale, N, acc_out);
    else
        hipLaunchKernelGGL((split_dequant<false>), fin, dim3(256), 0, s, Y, x_scale, w_scale, N, acc_out);
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
