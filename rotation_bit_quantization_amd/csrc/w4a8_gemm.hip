// spin_w4a8_gemm kernel: INT8 activations x INT4 weights -> int32 on the gfx950
// INT8 matrix cores, dequantised in the epilogue (the W4A8 setting that page
// "SpinQuant, Reproduced", Q7 lists among those the paper evaluates).
//
// The activation codes enter the MFMA as they are (one signed byte per code);
// the weight codes are widened from nibbles to 16 * code (gemm_common.h), so
// every product is 16 * qx * qw and the int32 sum is 16 times the true dot
// product (exact while 127 * 7 * 16 * K < 2^31); an arithmetic shift by 4
// recovers it.  The widening leaves the weight's k values in the order
// {0, 2, 4, 6}, {1, 3, 5, 7}, {8, ..., 14}, {9, ..., 15} within each group of 16,
// so each 16-byte activation fragment is permuted into that same order with
// four byte permutes.
//
// Tiles as in spin_w4a4_gemm: 256 x 256 per workgroup of 16 waves (4 x 4),
// 64 x 64 per wave as 2 x 2 tiles of the 32x32x32 int8 MFMA, operands streamed
// global -> LDS by DMA through a ring of stages, one barrier per step.  A step
// is 128 codes: 128 bytes per activation row and 64 per weight row, 48 KB per
// stage, three stages (the DMA runs two steps ahead).
//
// LDS layout of a stage: the 256 activation rows (128 bytes each, in groups of
// 8 rows = one DMA instruction), then the 256 weight rows (64 bytes, groups of
// 16 rows).  Activation row r keeps its logical 16-byte slot h at physical
// slot h ^ a_swz(r), a_swz(r) = (r ^ (r >> 3)) & 7, so that 16 consecutive rows
// reading one logical slot touch distinct banks; weight rows use slot_swz.
//
// Fragment k assignment (the same for both operands, so the sum over a step's
// 128 codes is unchanged): lane half L = lane / 32 and MFMA ks = 0..3 take
// codes 64 L + 16 ks .. 64 L + 16 ks + 15 of the step.
#include "gemm_common.h"
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

constexpr int kT8 = 256;                          // tile rows and columns
constexpr int kStep8 = 128;                       // codes per K step
constexpr int kRowA8 = 128;                       // bytes of an activation row per step
constexpr int kRowB8 = 64;                        // bytes of a weight row per step
constexpr int kStageA8 = kT8 * kRowA8;            // 32 KB
constexpr int kStage8 = kStageA8 + kT8 * kRowB8;  // 48 KB
constexpr int kStages8 = 3;
constexpr int kThreads8 = 1024;
constexpr int kD8 = 3;                            // DMA loads per wave per step: 2 A + 1 B

__device__ __forceinline__ int a_swz(int r) { return (r ^ (r >> 3)) & 7; }

// Activation bytes a0..a15 (natural k order) -> the order widen16 gives the
// weight codes: {a0, a2, a4, a6}, {a1, a3, a5, a7}, {a8, .., a14}, {a9, .., a15}.
__device__ __forceinline__ v4i perm_a16(uint4 q) {
    v4i r;
    r.x = static_cast<int>(__builtin_amdgcn_perm(q.y, q.x, 0x06040200u));
    r.y = static_cast<int>(__builtin_amdgcn_perm(q.y, q.x, 0x07050301u));
    r.z = static_cast<int>(__builtin_amdgcn_perm(q.w, q.z, 0x06040200u));
    r.w = static_cast<int>(__builtin_amdgcn_perm(q.w, q.z, 0x07050301u));
    return r;
}

template <bool WRITE_ACC>
__global__ __launch_bounds__(kThreads8) void w4a8_gemm_256(
    const int8_t* __restrict__ Xq8, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages8 * kStage8];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    int tm, tn;
    tile_of(blockIdx.x, (M + kT8 - 1) / kT8, (N + kT8 - 1) / kT8, &tm, &tn);
    const int m0 = tm * kT8, n0 = tn * kT8;
    const int wm = (wave >> 2) * 64, wn = (wave & 3) * 64;
    const size_t rowA = static_cast<size_t>(K), rowB = static_cast<size_t>(K) / 2;
    const int steps = K / kStep8;

    // DMA sources: activation groups g = wave and wave + 16 (8 rows each,
    // lane -> row 8 g + lane / 8, physical slot lane % 8), weight group wave
    // (16 rows, lane -> row 16 wave + lane / 4, physical slot lane % 4).
    // Rows past M or N read row 0 (valid memory) and are never stored.
    const uint8_t* ga[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = 8 * (wave + 16 * k) + (lane >> 3);
        const int h = (lane & 7) ^ a_swz(r);
        const int ra = m0 + r;
        ga[k] = reinterpret_cast<const uint8_t*>(Xq8) + static_cast<size_t>(ra < M ? ra : 0) * rowA + h * 16;
    }
    const uint8_t* gb;
    {
        const int r = 16 * wave + (lane >> 2);
        const int h = (lane & 3) ^ slot_swz(r);
        const int rb = n0 + r;
        gb = Wq + static_cast<size_t>(rb < N ? rb : 0) * rowB + h * 16;
    }
    const uint32_t lds0 = lds_addr(lds);
    auto issue = [&](int step) {
        const uint32_t stage = lds0 + (step % kStages8) * kStage8;
        const uint32_t a0 = __builtin_amdgcn_readfirstlane(stage + wave * 1024);
        const uint32_t b0 = __builtin_amdgcn_readfirstlane(stage + kStageA8 + wave * 1024);
        lds_dma16(ga[0] + static_cast<size_t>(step) * kRowA8, a0);
        lds_dma16(ga[1] + static_cast<size_t>(step) * kRowA8, a0 + 16 * 1024);
        lds_dma16(gb + static_cast<size_t>(step) * kRowB8, b0);
    };

    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // fragment offsets within a stage: activation rows r_i = wm + 32 i + lane % 32
    // at logical slot 4 L + ks; weight rows wn + 32 j + lane % 32 at logical
    // slot 2 L + part (two MFMAs per 16-byte read)
    const int fr = lane & 31, L = lane >> 5;
    int offa[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = wm + 32 * i + fr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) offa[i][ks] = r * kRowA8 + (((4 * L + ks) ^ a_swz(r)) << 4);
    }
    const int fob[2] = {fr * kRowB8 + (((2 * L) ^ slot_swz(fr)) << 4),
                        fr * kRowB8 + (((2 * L + 1) ^ slot_swz(fr)) << 4)};

#pragma unroll
    for (int s = 0; s < kStages8 - 1; ++s)
        if (s < steps) issue(s);
    // the epilogue's scales, requested now: thread t < 256 takes tile row t,
    // 256 <= t < 512 tile column t - 256
    float scale = 0.0f;
    if (tid < kT8) scale = x_scale[min(m0 + tid, M - 1)];
    else if (tid < 2 * kT8) scale = w_scale[min(n0 + tid - kT8, N - 1)];

    for (int step = 0; step < steps; ++step) {
        // This wave's loads of `step` are complete once at most the next
        // step's remain, and its LDS reads of the previous step are done; the
        // barrier then makes both hold for every wave, so the stage read last
        // step can be refilled.
        asm volatile("" ::: "memory");
        if (step + 1 < steps) __builtin_amdgcn_s_waitcnt(kD8 | 0x0070);
        else __builtin_amdgcn_s_waitcnt(0x0070);
        barrier_no_fence();
        if (step + kStages8 - 1 < steps) issue(step + kStages8 - 1);
        const uint8_t* st = lds + (step % kStages8) * kStage8;
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            uint4 qb[2], qa[2][2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                qb[j] = *reinterpret_cast<const uint4*>(st + kStageA8 + (wn + 32 * j) * kRowB8 + fob[part]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
                    qa[i][sub] = *reinterpret_cast<const uint4*>(st + offa[i][2 * part + sub]);
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                v4i fb[2];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    fb[j] = widen16(sub ? make_uint2(qb[j].z, qb[j].w) : make_uint2(qb[j].x, qb[j].y));
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const v4i fa = perm_a16(qa[i][sub]);
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, fb[j], acc[i][j], 0, 0, 0);
                }
            }
        }
    }

    // the tile's scales through LDS (read from global memory in the
    // epilogue, every store waited for its own two loads)
    const float* sc = stage_scales(lds, scale, tid < 2 * kT8);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float sx[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sx[r] = sc[wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = n0 + wn + j * 32 + (lane & 31);
                const int a = acc[i][j][r] >> 4;
                float y = static_cast<float>(a) * sx[r];
                y = y * sc[kT8 + wn + j * 32 + (lane & 31)];
                if (row < M && col < N) {
                    Y[static_cast<size_t>(row) * N + col] = y;
                    if (WRITE_ACC) acc_out[static_cast<size_t>(row) * N + col] = a;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_w4a8_gemm(const int8_t* Xq8, const float* x_scale, const uint8_t* Wq,
                            const float* w_scale, int M, int N, int K, float* Y,
                            int32_t* acc_out, hipStream_t s) {
    const long long tiles = static_cast<long long>((N + kT8 - 1) / kT8) * ((M + kT8 - 1) / kT8);
    dim3 grid(static_cast<unsigned>(tiles));
    if (acc_out)
        hipLaunchKernelGGL((w4a8_gemm_256<true>), grid, dim3(kThreads8), 0, s, Xq8, x_scale, Wq, w_scale, M,
                           N, K, Y, acc_out);
    else
        hipLaunchKernelGGL((w4a8_gemm_256<false>), grid, dim3(kThreads8), 0, s, Xq8, x_scale, Wq, w_scale, M,
                           N, K, Y, acc_out);
    return hipGetLastError();
}

}  // namespace spin
