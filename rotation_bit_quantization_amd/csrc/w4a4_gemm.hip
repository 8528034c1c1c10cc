// spin_w4a4_gemm kernel: INT4 x INT4 -> int32 on the gfx950 INT8 matrix cores,
// dequantised in the epilogue (abstract: W4A4; per-token activation scales and
// per-output-channel weight scales are this library's reading).
//
// Both operands are K-contiguous packed nibbles (activations [M][K/2], weights
// [N][K/2]).  CDNA4 has no INT4 matrix mode, so codes are widened to int8 in
// registers: masking a packed dword with 0xF0F0F0F0 leaves the odd codes in
// the high nibble of each byte, i.e. 16 * code as a signed byte, and shifting
// left by 4 first does the same for the even codes.  Both operands use the
// same widening, so every product is 256 * qx * qw and the int32 sum is 256
// times the true dot product (exact while 49 * K * 256 < 2^31); an arithmetic
// shift by 8 recovers it exactly.  The k order inside a 64-wide MFMA step is
// permuted identically on both sides, which leaves the dot product unchanged.
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBKBytes = 32;   // 64 codes per k-step

__device__ __forceinline__ v4i widen16(uint2 p) {
    v4i r;
    r.x = static_cast<int>((p.x << 4) & 0xF0F0F0F0u);
    r.y = static_cast<int>(p.x & 0xF0F0F0F0u);
    r.z = static_cast<int>((p.y << 4) & 0xF0F0F0F0u);
    r.w = static_cast<int>(p.y & 0xF0F0F0F0u);
    return r;
}

// 128 x 128 output tile per workgroup of 4 waves (2 x 2), 64 x 64 per wave as
// 4 x 4 MFMA 16x16x64 tiles.
template <bool WRITE_ACC>
__global__ __launch_bounds__(256) void w4a4_gemm_basic(
    const uint8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[kBM * kBKBytes];
    __shared__ __attribute__((aligned(16))) uint8_t sB[kBN * kBKBytes];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int tilesN = (N + kBN - 1) / kBN;
    const int m0 = static_cast<int>(blockIdx.x / tilesN) * kBM;
    const int n0 = static_cast<int>(blockIdx.x % tilesN) * kBN;
    const int wm = (wave >> 1) * 64;
    const int wn = (wave & 1) * 64;
    const size_t rowBytes = static_cast<size_t>(K) / 2;

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int lr = tid >> 1;            // row of the tile this thread stages
    const int lo = (tid & 1) * 16;      // byte offset within the 32-byte k-step
    const bool aok = (m0 + lr) < M;
    const bool bok = (n0 + lr) < N;
    const uint8_t* ag = Xq + static_cast<size_t>(aok ? m0 + lr : 0) * rowBytes + lo;
    const uint8_t* bg = Wq + static_cast<size_t>(bok ? n0 + lr : 0) * rowBytes + lo;

    for (size_t kb = 0; kb < rowBytes; kb += kBKBytes) {
        uint4 va = aok ? *reinterpret_cast<const uint4*>(ag + kb) : make_uint4(0, 0, 0, 0);
        uint4 vb = bok ? *reinterpret_cast<const uint4*>(bg + kb) : make_uint4(0, 0, 0, 0);
        __syncthreads();
        *reinterpret_cast<uint4*>(sA + lr * kBKBytes + lo) = va;
        *reinterpret_cast<uint4*>(sB + lr * kBKBytes + lo) = vb;
        __syncthreads();
        v4i fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ra = wm + i * 16 + (lane & 15);
            const int rb = wn + i * 16 + (lane & 15);
            fa[i] = widen16(*reinterpret_cast<const uint2*>(sA + ra * kBKBytes + (lane >> 4) * 8));
            fb[i] = widen16(*reinterpret_cast<const uint2*>(sB + rb * kBKBytes + (lane >> 4) * 8));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }

    // Output layout of a 16x16 MFMA tile: lane l holds rows 4 * (l / 16) + r,
    // r = 0..3, of column l % 16.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn + j * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + i * 16 + (lane >> 4) * 4 + r;
                if (row < M && col < N) {
                    const int a = acc[i][j][r] >> 8;
                    float y = static_cast<float>(a) * x_scale[row];
                    y = y * w_scale[col];
                    Y[static_cast<size_t>(row) * N + col] = y;
                    if (WRITE_ACC) acc_out[static_cast<size_t>(row) * N + col] = a;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// w4a4_gemm_256: 256 x 256 output tile per workgroup of 8 waves (2 x 4), each
// wave 128 x 64 (8 x 4 MFMA 16x16x64 tiles, int32 accumulators in the
// accumulation registers), two waves per SIMD so that one wave's MFMAs run
// while the other waits on LDS or widens operands.  K advances 64 codes
// (32 bytes per row) per step; the next step's 16 KB of packed operands is
// fetched into registers while the current step runs from LDS, then written
// to the other half of a double-buffered LDS (2 x 16 KB): one barrier per
// step.  Tiles are assigned so that the workgroups running on one XCD
// (hardware places workgroup i on XCD i mod 8) cover a compact block of tile
// rows and columns, which keeps the operands they share in that XCD's L2.
constexpr int kT = 256;
constexpr int kStepBytes = 32;
constexpr int kStageBytes = 2 * kT * kStepBytes;   // A then B
constexpr int kGemmThreads = 512;

__device__ __forceinline__ void tile_of(int bid, int tilesM, int tilesN, int* tm, int* tn) {
    const int T = tilesM * tilesN;
    int t = bid;
    if ((T & 7) == 0) t = (bid & 7) * (T >> 3) + (bid >> 3);    // contiguous block per XCD
    constexpr int G = 4;                                        // tile rows per group
    const int group = t / (G * tilesN);
    const int first = group * G;
    const int rows = min(G, tilesM - first);
    const int r = t - group * G * tilesN;
    *tm = first + r % rows;
    *tn = r / rows;
}

template <bool WRITE_ACC>
__global__ __launch_bounds__(kGemmThreads) void w4a4_gemm_256(
    const uint8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    int tm, tn;
    tile_of(blockIdx.x, (M + kT - 1) / kT, (N + kT - 1) / kT, &tm, &tn);
    const int m0 = tm * kT, n0 = tn * kT;
    const int wm = (wave >> 2) * 128, wn = (wave & 3) * 64;
    const size_t rowBytes = static_cast<size_t>(K) / 2;
    const int steps = K / 64;

    // staging: thread t moves 16 bytes of row t / 2 of A (t < 512 covers all
    // 256 rows) and the same of B
    const int sr = tid >> 1, so = (tid & 1) * 16;
    const bool oka = (m0 + sr) < M, okb = (n0 + sr) < N;
    const uint8_t* ga = Xq + static_cast<size_t>(oka ? m0 + sr : 0) * rowBytes + so;
    const uint8_t* gb = Wq + static_cast<size_t>(okb ? n0 + sr : 0) * rowBytes + so;
    uint4 pa, pb;
    auto fetch = [&](int step) {
        const size_t off = static_cast<size_t>(step) * kStepBytes;
        pa = oka ? *reinterpret_cast<const uint4*>(ga + off) : make_uint4(0, 0, 0, 0);
        pb = okb ? *reinterpret_cast<const uint4*>(gb + off) : make_uint4(0, 0, 0, 0);
    };
    // LDS rows are 32 bytes = four 8-byte chunks; chunk c of row r is stored at
    // slot c ^ ((r >> 2) & 3) so that the fragment reads (16 rows, same chunk)
    // fall in distinct banks.
    const int sw_st = (sr >> 2) & 3, c0 = (tid & 1) * 2;
    const int st0 = sr * kStepBytes + ((c0 ^ sw_st) << 3), st1 = sr * kStepBytes + (((c0 + 1) ^ sw_st) << 3);
    auto stash = [&](int buf) {
        uint8_t* base = lds + buf * kStageBytes;
        *reinterpret_cast<uint2*>(base + st0) = make_uint2(pa.x, pa.y);
        *reinterpret_cast<uint2*>(base + st1) = make_uint2(pa.z, pa.w);
        *reinterpret_cast<uint2*>(base + kT * kStepBytes + st0) = make_uint2(pb.x, pb.y);
        *reinterpret_cast<uint2*>(base + kT * kStepBytes + st1) = make_uint2(pb.z, pb.w);
    };

    v4i acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    fetch(0);
    stash(0);
    __syncthreads();
    const int fr = lane & 15, fk = ((lane >> 4) ^ ((fr >> 2) & 3)) * 8;   // swizzled chunk
    for (int step = 0; step < steps; ++step) {
        const int buf = step & 1;
        if (step + 1 < steps) fetch(step + 1);
        const uint8_t* sa = lds + buf * kStageBytes + (wm + fr) * kStepBytes + fk;
        const uint8_t* sb = lds + buf * kStageBytes + kT * kStepBytes + (wn + fr) * kStepBytes + fk;
        v4i fb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = widen16(*reinterpret_cast<const uint2*>(sb + j * 16 * kStepBytes));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const v4i fa = widen16(*reinterpret_cast<const uint2*>(sa + i * 16 * kStepBytes));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa, fb[j], acc[i][j], 0, 0, 0);
        }
        if (step + 1 < steps) stash(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float sx[4];
        int rows[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            rows[r] = m0 + wm + i * 16 + (lane >> 4) * 4 + r;
            sx[r] = rows[r] < M ? x_scale[rows[r]] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn + j * 16 + (lane & 15);
            if (col >= N) continue;
            const float sw = w_scale[col];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (rows[r] < M) {
                    const int a = acc[i][j][r] >> 8;
                    float y = static_cast<float>(a) * sx[r];
                    y = y * sw;
                    Y[static_cast<size_t>(rows[r]) * N + col] = y;
                    if (WRITE_ACC) acc_out[static_cast<size_t>(rows[r]) * N + col] = a;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                            const float* w_scale, int M, int N, int K, float* Y,
                            int32_t* acc_out, hipStream_t s) {
    const long long tiles = static_cast<long long>((N + kT - 1) / kT) * ((M + kT - 1) / kT);
    dim3 grid(static_cast<unsigned>(tiles));
    if (acc_out)
        hipLaunchKernelGGL((w4a4_gemm_256<true>), grid, dim3(kGemmThreads), 0, s, Xq, x_scale, Wq,
                           w_scale, M, N, K, Y, acc_out);
    else
        hipLaunchKernelGGL((w4a4_gemm_256<false>), grid, dim3(kGemmThreads), 0, s, Xq, x_scale, Wq,
                           w_scale, M, N, K, Y, acc_out);
    return hipGetLastError();
}

}  // namespace spin
