// spin_fold_rotation kernels: W' = blockdiag(B, ..., B)^T W followed by
// per-output-channel INT4 (page "SpinQuant, Reproduced", Q1 and Q5: R1/R2 are
// merged into the adjacent weights, free at runtime; R4's inverse is merged
// into down_proj).  With rows rotated as x -> x B, the matching weight is
// B^T W, so (x B)(B^T W) = x W.
//
// This runs once per weight, offline; it is a float32 VALU GEMM (MFMA is kept
// for the INT4 product).  B is either the caller's R or the library Hadamard
// H_r / sqrt(r), whose entries are generated from their index bits.
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

constexpr int kTile = 64;
constexpr int kTileJ = 16;

// Entry B[j][i] of the rotation block.
template <bool HAD>
__device__ __forceinline__ float block_entry(const float* R, int r, int j, int i, int log2p,
                                             bool has12, float norm) {
    if (HAD) return hadamard_sign(static_cast<unsigned>(j), static_cast<unsigned>(i), log2p, has12) * norm;
    return R[static_cast<size_t>(j) * r + i];
}

// r % 64 == 0: a 64 x 64 output tile lies inside one diagonal block.
template <bool HAD>
__global__ __launch_bounds__(256) void fold_gemm_tiled(const float* __restrict__ W, int /* K */, int N,
                                                       const float* __restrict__ R, int r,
                                                       int log2p, int has12, float norm,
                                                       float* __restrict__ W_rot) {
    __shared__ float sB[kTileJ][kTile + 1];
    __shared__ float sW[kTileJ][kTile + 4];
    const int n0 = blockIdx.x * kTile;
    const int k0 = blockIdx.y * kTile;
    const int kb = (k0 / r) * r;   // first row of the diagonal block
    const int i0 = k0 - kb;        // first local output index of the tile
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    float acc[4][4] = {};
    for (int j0 = 0; j0 < r; j0 += kTileJ) {
        for (int e = tid; e < kTileJ * kTile; e += 256) {
            const int jj = e / kTile, ii = e % kTile;
            sB[jj][ii] = block_entry<HAD>(R, r, j0 + jj, i0 + ii, log2p, has12 != 0, norm);
            const int col = n0 + ii;
            sW[jj][ii] = (col < N) ? W[static_cast<size_t>(kb + j0 + jj) * N + col] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < kTileJ; ++jj) {
            float bi[4], wn[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bi[q] = sB[jj][ty * 4 + q];
                wn[q] = sW[jj][tx * 4 + q];
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(bi[a], wn[b], acc[a][b]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const size_t rowoff = static_cast<size_t>(k0 + ty * 4 + a) * N;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = n0 + tx * 4 + b;
            if (col < N) W_rot[rowoff + col] = acc[a][b];
        }
    }
}

// Any r: one output element per thread.
template <bool HAD>
__global__ __launch_bounds__(256) void fold_gemm_simple(const float* __restrict__ W, int K, int N,
                                                        const float* __restrict__ R, int r,
                                                        int log2p, int has12, float norm,
                                                        float* __restrict__ W_rot) {
    const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<size_t>(K) * N) return;
    const int k = static_cast<int>(idx / N);
    const int n = static_cast<int>(idx % N);
    const int kb = (k / r) * r;
    const int i = k - kb;
    float acc = 0.0f;
    for (int j = 0; j < r; ++j)
        acc = __builtin_fmaf(block_entry<HAD>(R, r, j, i, log2p, has12 != 0, norm),
                             W[static_cast<size_t>(kb + j) * N + n], acc);
    W_rot[idx] = acc;
}

// Per-column absmax scale, then codes packed output-channel-major [N][K/2].
// One workgroup per 64 columns; K is walked in 64-row tiles staged in LDS so
// that each thread writes 16 consecutive codes (8 bytes) of one column.
__global__ __launch_bounds__(256) void fold_quant(const float* __restrict__ W_rot, int K, int N,
                                                  uint8_t* __restrict__ Wq,
                                                  float* __restrict__ w_scale) {
    __shared__ float tile[kTile][kTile + 1];
    __shared__ float red[4][kTile];
    __shared__ float sS[kTile];
    const int n0 = blockIdx.x * kTile;
    const int tid = threadIdx.x;
    const int tn = tid & 63, tk = tid >> 6;
    const int col = n0 + tn;
    float mx = 0.0f;
    if (col < N)
        for (int k = tk; k < K; k += 4)
            mx = __builtin_fmaxf(mx, __builtin_fabsf(W_rot[static_cast<size_t>(k) * N + col]));
    red[tk][tn] = mx;
    __syncthreads();
    if (tk == 0) {
        const float a = __builtin_fmaxf(__builtin_fmaxf(red[0][tn], red[1][tn]),
                                        __builtin_fmaxf(red[2][tn], red[3][tn]));
        const float s = __fdiv_rn(a, kSeven);
        sS[tn] = s;
        if (col < N) w_scale[col] = s;
    }
    const int nl = tid >> 2, kq = tid & 3;
    for (int kc = 0; kc < K; kc += kTile) {
        __syncthreads();
        for (int e = tid; e < kTile * kTile; e += 256) {
            const int kk = e / kTile, nn = e % kTile;
            tile[kk][nn] = (n0 + nn < N) ? W_rot[static_cast<size_t>(kc + kk) * N + n0 + nn] : 0.0f;
        }
        __syncthreads();
        if (n0 + nl < N) {
            const float s = sS[nl];
            int c[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) c[j] = quant_exact(tile[kq * 16 + j][nl], s);
            uint2 w;
            w.x = pack8(c);
            w.y = pack8(c + 8);
            *reinterpret_cast<uint2*>(Wq + static_cast<size_t>(n0 + nl) * (K / 2) + (kc + kq * 16) / 2) = w;
        }
    }
}

template <bool HAD>
hipError_t launch_gemm(const float* W, int K, int N, const float* R, int r, HadOrder h,
                       float* W_rot, hipStream_t s) {
    const float norm = HAD ? static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(r))) : 1.0f;
    if (r % kTile == 0) {
        dim3 grid((N + kTile - 1) / kTile, K / kTile);
        hipLaunchKernelGGL((fold_gemm_tiled<HAD>), grid, dim3(256), 0, s, W, K, N, R, r, h.log2p,
                           h.has12 ? 1 : 0, norm, W_rot);
    } else {
        const size_t total = static_cast<size_t>(K) * N;
        hipLaunchKernelGGL((fold_gemm_simple<HAD>), dim3(static_cast<unsigned>((total + 255) / 256)),
                           dim3(256), 0, s, W, K, N, R, r, h.log2p, h.has12 ? 1 : 0, norm, W_rot);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fold_rotation(const float* W, int K, int N, const float* R, int r_block,
                                HadOrder h, float* W_rot, uint8_t* Wq, float* w_scale,
                                hipStream_t s) {
    hipError_t e = R ? launch_gemm<false>(W, K, N, R, r_block, h, W_rot, s)
                     : launch_gemm<true>(W, K, N, R, r_block, h, W_rot, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fold_quant, dim3((N + kTile - 1) / kTile), dim3(256), 0, s, W_rot, K, N,
                       Wq, w_scale);
    return hipGetLastError();
}

}  // namespace spin
