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

template <bool WRITE_ACC>
__global__ __launch_bounds__(kF6Threads) void w4a4_gemm_fp6_f6ab(
    const uint8_t* __restrict__ Xf6, const int32_t* __restrict__ x_sum, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wf6, const int32_t* __restrict__ w_sum, const float* __restrict__ w_scale, int M,
    int N, int K, float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * kF6StageBytes];
    int tm, tn;
    tile_of(blockIdx.x, (M + kF6T - 1) / kF6T, (N + kF6T - 1) / kF6T, &tm, &tn);
    gemm_tile_f6ab<WRITE_ACC>(Xf6, x_sum, x_scale, Wf6, w_sum, w_scale, M, N, K, Y, acc_out, tm, tn, lds);
}

// Packed codes [N][K/2] -> the FP6 operand layout (the conversion the
// tiles apply to 16-byte chunks, so that the fields and their order are the
// ones the tiles would have written to their stages) and the code sum of
// every row.  Workgroup b takes the 32-row block b; its sixteen waves split
// the block's 64-code k-steps in sixteen.  For each k-step lane l converts k-half
// l / 32 of row l % 32, so that the wave writes the step's 1536-byte region
// whole; the row sums are reduced in the LDS.  Rows past N are not written.
constexpr int kCodesWaves = 16;

__global__ __launch_bounds__(64 * kCodesWaves) void codes_f6_kernel(const uint8_t* __restrict__ Wq, int N, int K,
                                                       uint8_t* __restrict__ Wf6, int32_t* __restrict__ w_sum) {
    const int blk = static_cast<int>(blockIdx.x);
    const int wave = static_cast<int>(threadIdx.x >> 6), lane = static_cast<int>(threadIdx.x & 63);
    const int r = lane & 31, h = lane >> 5;
    const int row = 32 * blk + r;
    const bool live = row < N;
    const int ksteps = K / 64;
    const int k0 = wave * ksteps / kCodesWaves, k1 = (wave + 1) * ksteps / kCodesWaves;
    const uint8_t* src = Wq + static_cast<size_t>(live ? row : 0) * (K / 2) + 16 * h;
    uint8_t* dst = Wf6 + static_cast<size_t>(blk) * ksteps * 1536 + h * 768 + r * 24;
    int sum = 0;
#pragma unroll 4
    for (int ks = k0; ks < k1; ++ks) {
        const uint4 q = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(ks) * 32);
        uint32_t o[6];
        chunk_to_fp6(q, o, sum);
        if (live) {
            uint2* d = reinterpret_cast<uint2*>(dst + static_cast<size_t>(ks) * 1536);
            d[0] = make_uint2(o[0], o[1]);
            d[1] = make_uint2(o[2], o[3]);
            d[2] = make_uint2(o[4], o[5]);
        }
    }
    sum += __shfl_xor(sum, 32, 64);   // the row's two k-halves
    __shared__ int part[kCodesWaves][32];
    if (h == 0) part[wave][r] = sum;
    __syncthreads();
    if (threadIdx.x < 32 && 32 * blk + static_cast<int>(threadIdx.x) < N) {
        int t = 0;
#pragma unroll
        for (int w = 0; w < kCodesWaves; ++w) t += part[w][threadIdx.x];
        w_sum[32 * blk + threadIdx.x] = t;
    }
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

// Zeroes n words of the 16-byte-aligned p (a kernel rather than a memset, so
// that the three launches of a split product can be captured in a graph).
__global__ __launch_bounds__(256) void zero_partials(uint32_t* __restrict__ p, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    const size_t i0 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint4* q = reinterpret_cast<uint4*>(p);
    for (size_t i = i0; i < n / 4; i += stride) q[i] = make_uint4(0, 0, 0, 0);
    if (i0 < n % 4) p[n / 4 * 4 + i0] = 0;
}

// Row blockIdx.x of the summed int32 accumulators in Y -> the dequantized
// float32 outputs, in place, with the epilogue arithmetic of the tile; VEC4:
// four columns per thread (N % 4 == 0, every row 16-byte aligned).
template <bool WRITE_ACC, bool VEC4>
__global__ __launch_bounds__(256) void split_dequant(float* __restrict__ Y, const float* __restrict__ x_scale,
                                                     const float* __restrict__ w_scale, int N,
                                                     int32_t* __restrict__ acc_out) {
    const int row = static_cast<int>(blockIdx.x);
    const float sx = x_scale[row];
    const size_t base = static_cast<size_t>(row) * N;
    auto one = [&](uint32_t word, float sw, float& y, int& a) {
        a = static_cast<int>(word);
        y = static_cast<float>(a) * sx;
        y = y * sw;
    };
    if constexpr (VEC4) {
        for (int c = static_cast<int>(blockIdx.y * blockDim.x + threadIdx.x); 4 * c < N;
             c += static_cast<int>(gridDim.y * blockDim.x)) {
            const uint4 w = *reinterpret_cast<const uint4*>(Y + base + 4 * c);
            const float4 sw = *reinterpret_cast<const float4*>(w_scale + 4 * c);
            float4 y;
            int4 a;
            one(w.x, sw.x, y.x, a.x);
            one(w.y, sw.y, y.y, a.y);
            one(w.z, sw.z, y.z, a.z);
            one(w.w, sw.w, y.w, a.w);
            *reinterpret_cast<float4*>(Y + base + 4 * c) = y;
            if (WRITE_ACC) *reinterpret_cast<int4*>(acc_out + base + 4 * c) = a;
        }
    } else {
        for (int col = static_cast<int>(blockIdx.y * blockDim.x + threadIdx.x); col < N;
             col += static_cast<int>(gridDim.y * blockDim.x)) {
            float y;
            int a;
            one(__builtin_bit_cast(uint32_t, Y[base + col]), w_scale[col], y, a);
            Y[base + col] = y;
            if (WRITE_ACC) acc_out[base + col] = a;
        }
    }
}

template <bool WRITE_ACC>
void launch_dequant(dim3 grid, bool vec4, hipStream_t s, float* Y, const float* x_scale, const float* w_scale,
                    int N, int32_t* acc_out) {
    if (vec4)
        hipLaunchKernelGGL((split_dequant<WRITE_ACC, true>), grid, dim3(256), 0, s, Y, x_scale, w_scale, N, acc_out);
    else
        hipLaunchKernelGGL((split_dequant<WRITE_ACC, false>), grid, dim3(256), 0, s, Y, x_scale, w_scale, N, acc_out);
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

// Number of K slices for the split-K form, 0 where it does not apply.  The
// costs are fits to MI355X timings (µs, outputs in millions):
//   slices       1.35 per step of 128 codes in the longest slice, plus 2.8 per
//                million atomic int32 additions (slices x outputs; the
//                additions are bound by their bytes: packing two outputs into
//                one 64-bit addition measured no faster);
//   fill + pass  8 + 1.9 per million outputs (two short launches);
//   whole tiles  16 + 1.17 per step, plus 0.0018 per step and tile (one round
//                of the int8 or FP6 256 x 256 tiles: the alternative).
// The slice count is the power of two that minimises the slices' cost while
// every slice keeps two steps or more and all slices fit in one round of the
// compute units.  AUTO takes it only past the weight-streaming kernel's 128
// rows, where the whole tiles leave half of the compute units idle, and when
// the prediction is at least 5% below the whole tiles'.
int w4a4_gemm_fp6_split_slices(int M, int N, int K, bool forced) {
    if (M <= 0 || N <= 0 || K % kF6StepCodes != 0 || K < 2 * kF6StepCodes || K > kGemmFp6MaxK) return 0;
    const int cus = device_cu_count();
    if (cus <= 0) return 0;
    const long long tiles = static_cast<long long>((M + kF6T - 1) / kF6T) * ((N + kF6T - 1) / kF6T);
    if (!forced && (M <= 128 || 2 * tiles > cus)) return 0;
    const int steps = K / kF6StepCodes;
    const double outputs = static_cast<double>(M) * N / 1e6;
    auto cost = [&](int S) { return 1.35 * ((steps + S - 1) / S) + 2.8 * S * outputs; };
    int best = 1;
    for (int S = 2; steps / S >= 2 && tiles * S <= cus; S *= 2)
        if (cost(S) < cost(best)) best = S;
    if (forced) return best;
    const double whole = 16.0 + 1.17 * steps + 0.0018 * steps * static_cast<double>(tiles);
    const double split = cost(best) + 8.0 + 1.9 * outputs;
    return best >= 2 && split < 0.95 * whole ? best : 0;
}

hipError_t launch_w4a4_gemm_fp6_split(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                                      const float* w_scale, int M, int N, int K, int slices, float* Y,
                                      int32_t* acc_out, hipStream_t s) {
    if (K % kF6StepCodes != 0 || K < 2 * kF6StepCodes || K > kGemmFp6MaxK || slices < 1 ||
        K / kF6StepCodes < 2 * slices)
        return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    const size_t n = static_cast<size_t>(M) * N;
    const unsigned zb = static_cast<unsigned>(std::min<size_t>((n / 4 + 255) / 256 + 1, 8192));
    hipLaunchKernelGGL(zero_partials, dim3(zb), dim3(256), 0, s, reinterpret_cast<uint32_t*>(Y), n);
    const long long tiles = static_cast<long long>((M + kF6T - 1) / kF6T) * ((N + kF6T - 1) / kF6T);
    hipLaunchKernelGGL(w4a4_gemm_fp6_split, dim3(static_cast<unsigned>(tiles * slices)), dim3(kF6Threads), 0, s,
                       Xq, Wq, M, N, K, slices, Y);
    const bool vec4 = N % 4 == 0;
    const dim3 fin(static_cast<unsigned>(M), static_cast<unsigned>((N + (vec4 ? 1023 : 255)) / (vec4 ? 1024 : 256)));
    if (acc_out)
        launch_dequant<true>(fin, vec4, s, Y, x_scale, w_scale, N, acc_out);
    else
        launch_dequant<false>(fin, vec4, s, Y, x_scale, w_scale, N, acc_out);
    return hipGetLastError();
}

hipError_t launch_codes_f6(const uint8_t* Wq, int N, int K, uint8_t* Wf6, int32_t* w_sum, hipStream_t s) {
    if (N <= 0 || K % 64 != 0 || K <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(codes_f6_kernel, dim3(static_cast<unsigned>((N + 31) / 32)), dim3(64 * kCodesWaves), 0, s, Wq,
                       N, K, Wf6, w_sum);
    return hipGetLastError();
}

hipError_t launch_w4a4_gemm_f6f6(const uint8_t* Xf6, const int32_t* x_sum, const float* x_scale,
                                 const uint8_t* Wf6, const int32_t* w_sum, const float* w_scale, int M, int N, int K,
                                 float* Y, int32_t* acc_out, hipStream_t s) {
    if (K % kF6StepCodes != 0 || K < 2 * kF6StepCodes || K > kGemmFp6MaxK) return hipErrorInvalidValue;
    const long long tiles = static_cast<long long>((M + kF6T - 1) / kF6T) * ((N + kF6T - 1) / kF6T);
    const dim3 grid(static_cast<unsigned>(tiles));
    if (acc_out)
        hipLaunchKernelGGL((w4a4_gemm_fp6_f6ab<true>), grid, dim3(kF6Threads), 0, s, Xf6, x_sum, x_scale, Wf6, w_sum,
                           w_scale, M, N, K, Y, acc_out);
    else
        hipLaunchKernelGGL((w4a4_gemm_fp6_f6ab<false>), grid, dim3(kF6Threads), 0, s, Xf6, x_sum, x_scale, Wf6,
                           w_sum, w_scale, M, N, K, Y, acc_out);
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
