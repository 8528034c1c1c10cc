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
//
// Kernels: w4a4_gemm_256 (256 x 256 tiles, the general case), w4a4_gemm_wide
// (256 x 384 tiles where they fill the last round of workgroups better),
// w4a4_gemm_m16 (M <= 128, weight-streaming) and w4a4_gemm_basic (K not a
// multiple of 128).
#include "gemm_common.h"
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBKBytes = 32;   // 64 codes per k-step

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
    // r = 0..3, of column l % 16.  The scales are loaded ahead of the stores'
    // branches (inside them every store would wait for its own loads).
    float sw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sw[j] = w_scale[min(n0 + wn + j * 16 + (lane & 15), N - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sx[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sx[r] = x_scale[min(m0 + wm + i * 16 + (lane >> 4) * 4 + r, M - 1)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn + j * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + i * 16 + (lane >> 4) * 4 + r;
                if (row < M && col < N) {
                    const int a = acc[i][j][r] >> 8;
                    float y = static_cast<float>(a) * sx[r];
                    y = y * sw[j];
                    Y[static_cast<size_t>(row) * N + col] = y;
                    if (WRITE_ACC) acc_out[static_cast<size_t>(row) * N + col] = a;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// w4a4_gemm_256: 256 x 256 output tile per workgroup of 16 waves (4 x 4), each
// wave 64 x 64 as 2 x 2 tiles of the 32x32x32 int8 MFMA (the 32x32 shape
// sustains a higher int8 rate on gfx950 than 16x16x64), four waves per SIMD so
// that LDS latency and the per-step barrier are hidden behind other waves.
//
// Operands stream from global memory straight into LDS (global_load_lds, 16
// bytes per lane) through a ring of kStages LDS stages of one K step each
// (128 codes = 64 bytes per row; 32 KB per stage).  Loads run kStages - 1
// steps ahead of the MFMAs, with one barrier per step and explicit
// vector-memory waits (a full workgroup fence would drain every load in
// flight).  These loads are issued from assembly: the compiler would
// otherwise wait for all of them before every LDS read.
//
// LDS layout of a stage: for A then B, 8 blocks of 32 rows (2 KB each, one DMA
// instruction from each of two waves); inside a block the 16-byte slot 4 r + p holds
// logical slot h = p ^ f(r) of row r, f(r) = ((r >> 1) ^ (r >> 3)) & 3, so that
// 16-byte reads of one logical slot by 8 (or 16) consecutive rows touch
// distinct banks.
//
// MFMA 32x32x32 operand layout used here: lane l supplies row (or column)
// l % 32 and 16 k values; lanes 0-31 take logical slots 0-1 of the step,
// lanes 32-63 slots 2-3, and the four MFMAs of a step take bytes 0-7 and 8-15
// of the lane's first slot, then of its second (the same assignment for A
// and B, so the sum over the 128 codes is unchanged).  Result register r of
// lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4 of column l % 32.
//
// Rows beyond M or N load row 0 instead (any valid data); their results are
// never stored.  Tiles are assigned so that the workgroups running on one XCD
// (hardware places workgroup i on XCD i mod 8) cover a compact block of tile
// rows and columns, which keeps the operands they share in that XCD's L2.
constexpr int kT = 256;
constexpr int kStepCodes = 128;
constexpr int kStepBytes = kStepCodes / 2;
constexpr int kStageBytes = 2 * kT * kStepBytes;   // A then B
constexpr int kStages = 4;
constexpr int kGemmThreads = 1024;

template <bool WRITE_ACC>
__global__ __launch_bounds__(kGemmThreads) void w4a4_gemm_256(
    const uint8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStageBytes];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    int tm, tn;
    tile_of(blockIdx.x, (M + kT - 1) / kT, (N + kT - 1) / kT, &tm, &tn);
    const int m0 = tm * kT, n0 = tn * kT;
    const int wm = (wave >> 2) * 64, wn = (wave & 3) * 64;
    const size_t rowBytes = static_cast<size_t>(K) / 2;
    const int steps = K / kStepCodes;

    // DMA source of this lane: the wave fills rows 16 (wave & 1) .. + 15 of the
    // 32-row block wave / 2; 16-byte slot q = 64 (wave & 1) + lane of the block
    // = row q / 4, physical slot q % 4
    const uint8_t* ga;
    const uint8_t* gb;
    {
        const int q = 64 * (wave & 1) + lane;
        const int r = q >> 2;
        const int h = (q & 3) ^ slot_swz(r);
        const int ra = m0 + 32 * (wave >> 1) + r, rb = n0 + 32 * (wave >> 1) + r;
        ga = Xq + static_cast<size_t>(ra < M ? ra : 0) * rowBytes + h * 16;
        gb = Wq + static_cast<size_t>(rb < N ? rb : 0) * rowBytes + h * 16;
    }
    const uint32_t lds_wave = lds_addr(lds) + wave * 1024;
    auto issue = [&](int step) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_wave + (step % kStages) * kStageBytes);
        const size_t off = static_cast<size_t>(step) * kStepBytes;
        lds_dma16(ga + off, base);
        lds_dma16(gb + off, base + kT * kStepBytes);
    };

    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // fragment reads: row l % 32 of a 32-row block, logical slots 2 (l / 32)
    // and 2 (l / 32) + 1
    const int fr = lane & 31;
    const int h0 = 2 * (lane >> 5);
    const int fo0 = fr * kStepBytes + ((h0 ^ slot_swz(fr)) << 4);
    const int fo1 = fr * kStepBytes + (((h0 + 1) ^ slot_swz(fr)) << 4);

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < steps) issue(s);
    // the epilogue's scales, requested now: thread t < 256 takes tile row t,
    // 256 <= t < 512 tile column t - 256
    float scale = 0.0f;
    if (tid < kT) scale = x_scale[min(m0 + tid, M - 1)];
    else if (tid < 2 * kT) scale = w_scale[min(n0 + tid - kT, N - 1)];

    for (int step = 0; step < steps; ++step) {
        // This wave's loads of `step` are done once at most (later steps in
        // flight) x 4 remain; the barrier then also guarantees that every
        // wave has finished reading the stage refilled below.
        const int later = min(kStages - 2, steps - 1 - step);
        if (later >= 2) SPIN_WAIT_VMCNT(4);
        else if (later == 1) SPIN_WAIT_VMCNT(2);
        else SPIN_WAIT_VMCNT(0);
        barrier_no_fence();
        if (step + kStages - 1 < steps) issue(step + kStages - 1);
        const uint8_t* st = lds + (step % kStages) * kStageBytes;
        // all fragments of the step first, then the MFMAs ordered so that
        // consecutive ones never update the same accumulator
        uint4 qa[2][2], qb[2][2];
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            const int fo = part ? fo1 : fo0;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                qb[part][j] = *reinterpret_cast<const uint4*>(st + kT * kStepBytes + (wn + j * 32) * kStepBytes + fo);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                qa[part][i] = *reinterpret_cast<const uint4*>(st + (wm + i * 32) * kStepBytes + fo);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int part = ks >> 1, sub = ks & 1;
            v4i fb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                fb[j] = widen16(sub ? make_uint2(qb[part][j].z, qb[part][j].w)
                                    : make_uint2(qb[part][j].x, qb[part][j].y));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const v4i fa = widen16(sub ? make_uint2(qa[part][i].z, qa[part][i].w)
                                           : make_uint2(qa[part][i].x, qa[part][i].y));
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, fb[j], acc[i][j], 0, 0, 0);
            }
        }
    }

    // the tile's scales through LDS (read from global memory in the
    // epilogue, every store waited for its own two loads)
    const float* sc = stage_scales(lds, scale, tid < 2 * kT);
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
                const int a = acc[i][j][r] >> 8;
                float y = static_cast<float>(a) * sx[r];
                y = y * sc[kT + wn + j * 32 + (lane & 31)];
                if (row < M && col < N) {
                    Y[static_cast<size_t>(row) * N + col] = y;
                    if (WRITE_ACC) acc_out[static_cast<size_t>(row) * N + col] = a;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// w4a4_gemm_wide: 256 x 384 output tiles for shapes whose 256 x 256 tiles
// would leave the last round of workgroups part-empty (qkv_proj, N = 6144:
// 384 tiles of 256 x 256 on 256 CUs, 256 of 256 x 384).  Eight waves (two per
// SIMD), each 128 x 96 as 4 x 3 tiles of the 32x32x32 int8 MFMA; the same
// widening, LDS-DMA operand pipeline (three 40 KB stages, two steps ahead),
// slot swizzle, fragment layout and epilogue as w4a4_gemm_256.  A stage holds
// A's 8 and then B's 12 blocks of 32 rows; each wave issues five of its forty
// 1 KB DMA instructions (instruction q fills half q % 2 of block q / 2), from
// the block's wave-uniform row base plus the lane's offset in the block.  Only
// launched for whole tiles (M % 256 == 0, N % 384 == 0).
constexpr int kWTM = 256;
constexpr int kWTN = 384;
constexpr int kWStageBytes = (kWTM + kWTN) * kStepBytes;
constexpr int kWStages = 3;
constexpr int kWThreads = 512;
constexpr int kWDma = (kWTM + kWTN) * kStepBytes / 1024 / (kWThreads / 64);
static_assert(kWDma * 1024 * (kWThreads / 64) == kWStageBytes, "DMA instructions must tile a stage");

// 16 bytes per lane from sbase + voff into LDS at lds_base + 16 * lane, with
// a wave-uniform 64-bit base in scalar registers and a 32-bit per-lane offset
// (the same M0 handling as lds_dma16).
__device__ __forceinline__ void lds_dma16_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
        : "memory");
}

template <bool WRITE_ACC>
__global__ __launch_bounds__(kWThreads) void w4a4_gemm_wide(
    const uint8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kWStages * kWStageBytes];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    int tm, tn;
    tile_of(blockIdx.x, (M + kWTM - 1) / kWTM, (N + kWTN - 1) / kWTN, &tm, &tn);
    const int m0 = tm * kWTM, n0 = tn * kWTN;
    const int wm = (wave >> 2) * 128, wn = (wave & 3) * 96;
    const size_t rowBytes = static_cast<size_t>(K) / 2;
    const int steps = K / kStepCodes;

    // a lane's byte offset inside a 32-row block for each half (the row and
    // its swizzled 16-byte slot); the block's row base is wave-uniform and
    // goes in as the scalar base of the load
    uint32_t voff[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int r = 16 * half + (lane >> 2);
        voff[half] = static_cast<uint32_t>(r * rowBytes + ((lane & 3) ^ slot_swz(r)) * 16);
    }
    const uint32_t lds0 = lds_addr(lds);
    auto issue = [&](int step) {
        const uint32_t stage = lds0 + (step % kWStages) * kWStageBytes;
        const size_t off = static_cast<size_t>(step) * kStepBytes;
#pragma unroll
        for (int k = 0; k < kWDma; ++k) {
            const int q = __builtin_amdgcn_readfirstlane(kWDma * wave + k);
            const int blk = q >> 1, half = q & 1;
            const uint8_t* base = blk < kWTM / 32 ? Xq + static_cast<size_t>(m0 + 32 * blk) * rowBytes
                                                  : Wq + static_cast<size_t>(n0 + 32 * (blk - kWTM / 32)) * rowBytes;
            lds_dma16_s(voff[half], base + off, stage + blk * 2048 + half * 1024);
        }
    };

    v16i acc[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int fr = lane & 31;
    const int h0 = 2 * (lane >> 5);
    const int fo0 = fr * kStepBytes + ((h0 ^ slot_swz(fr)) << 4);
    const int fo1 = fr * kStepBytes + (((h0 + 1) ^ slot_swz(fr)) << 4);

#pragma unroll
    for (int s = 0; s < kWStages - 1; ++s)
        if (s < steps) issue(s);

    for (int step = 0; step < steps; ++step) {
        // this wave's loads of `step` are done once at most those of the one
        // later step in flight remain; the barrier then also guarantees that
        // every wave has finished reading the stage refilled below
        if (step + 1 < steps) SPIN_WAIT_VMCNT(kWDma);
        else SPIN_WAIT_VMCNT(0);
        barrier_no_fence();
        if (step + kWStages - 1 < steps) issue(step + kWStages - 1);
        const uint8_t* st = lds + (step % kWStages) * kWStageBytes;
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            const int fo = part ? fo1 : fo0;
            uint4 qa[4], qb[3];
#pragma unroll
            for (int j = 0; j < 3; ++j)
                qb[j] = *reinterpret_cast<const uint4*>(st + kWTM * kStepBytes + (wn + j * 32) * kStepBytes + fo);
#pragma unroll
            for (int i = 0; i < 4; ++i) qa[i] = *reinterpret_cast<const uint4*>(st + (wm + i * 32) * kStepBytes + fo);
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                v4i fb[3];
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    fb[j] = widen16(sub ? make_uint2(qb[j].z, qb[j].w) : make_uint2(qb[j].x, qb[j].y));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v4i fa = widen16(sub ? make_uint2(qa[i].z, qa[i].w) : make_uint2(qa[i].x, qa[i].y));
#pragma unroll
                    for (int j = 0; j < 3; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, fb[j], acc[i][j], 0, 0, 0);
                }
            }
        }
    }

    // the tile's 256 row and 384 column scales through LDS (whole tiles: every
    // index is in range), loaded once here rather than one store at a time
    {
        const float v0 = tid < kWTM ? x_scale[m0 + tid] : w_scale[n0 + tid - kWTM];
        const float v1 = tid < kWTN + kWTM - kWThreads ? w_scale[n0 + kWThreads - kWTM + tid] : 0.0f;
        float* sc = reinterpret_cast<float*>(lds);
        __syncthreads();
        sc[tid] = v0;
        if (tid < kWTN + kWTM - kWThreads) sc[kWThreads + tid] = v1;
        __syncthreads();
    }
    const float* sc = reinterpret_cast<const float*>(lds);
    float sw[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) sw[j] = sc[kWTM + wn + j * 32 + (lane & 31)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sx[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sx[r] = sc[wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int col = n0 + wn + j * 32 + (lane & 31);
                const int a = acc[i][j][r] >> 8;
                float y = static_cast<float>(a) * sx[r];
                y = y * sw[j];
                Y[static_cast<size_t>(row) * N + col] = y;
                if (WRITE_ACC) acc_out[static_cast<size_t>(row) * N + col] = a;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// w4a4_gemm_m16: M <= 128 (decode, short prompts), where the product is bound by reading
// the weights once.  One workgroup per 16 output columns; its waves (8, or 2
// when there are enough column groups to fill the chip) split K into ranges
// of 128-code chunks.  For each of the RG groups of 16 rows a wave runs two
// 16x16x64 int8 MFMA chains over its range (lane l: row / column l % 16, 16
// bytes at offset 16 (l / 16) of each 64-byte chunk, the MFMA pair taking bytes
// 0-7 then 8-15, identically for both operands); every weight chunk loaded
// serves all RG row groups.  The partial accumulators are added exactly in
// LDS.  Rows beyond M and columns beyond N read the last row / column (valid
// memory) and are never stored.
template <bool WRITE_ACC, int kDecodeWaves, int RG>
__global__ __launch_bounds__(64 * kDecodeWaves) void w4a4_gemm_m16(
    const uint8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ v4i part[kDecodeWaves][RG][64];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n0 = blockIdx.x * 16;
    const int cb = min(n0 + (lane & 15), N - 1);
    const size_t rowBytes = static_cast<size_t>(K) / 2;
    const uint8_t* pa[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g)
        pa[g] = Xq + static_cast<size_t>(min(16 * g + (lane & 15), M - 1)) * rowBytes + 16 * (lane >> 4);
    const uint8_t* pb = Wq + static_cast<size_t>(cb) * rowBytes + 16 * (lane >> 4);
    // the epilogue's scales, requested before the operands so that their
    // latency hides behind the main loads
    const int col = n0 + (lane & 15);
    const float sw = w_scale[cb];
    float sx[RG][4];
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) sx[g][r] = x_scale[min(16 * g + (lane >> 4) * 4 + r, M - 1)];
    const int chunks = K / 128;
    const int beg = (chunks * wave) / kDecodeWaves, end = (chunks * (wave + 1)) / kDecodeWaves;
    v4i acc0[RG], acc1[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) acc0[g] = acc1[g] = v4i{0, 0, 0, 0};
    // Chunks in groups of U with every load of a group issued before its
    // MFMAs (written out: the matrix builtins are convergent, so the compiler
    // does not unroll a loop with a run-time trip count around them), then
    // the remainder one at a time; beg and end are uniform across the wave.
    constexpr int U = RG == 1 ? 4 : RG <= 2 ? 2 : 1;
    auto step = [&](const uint4& qb, const uint4* qa) {
        const v4i b0 = widen16(make_uint2(qb.x, qb.y)), b1 = widen16(make_uint2(qb.z, qb.w));
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            acc0[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen16(make_uint2(qa[g].x, qa[g].y)), b0, acc0[g], 0, 0, 0);
            acc1[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen16(make_uint2(qa[g].z, qa[g].w)), b1, acc1[g], 0, 0, 0);
        }
    };
    int it = beg;
    for (; it + U <= end; it += U) {
        uint4 qb[U], qa[U][RG];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            qb[u] = *reinterpret_cast<const uint4*>(pb + static_cast<size_t>(it + u) * 64);
#pragma unroll
            for (int g = 0; g < RG; ++g)
                qa[u][g] = *reinterpret_cast<const uint4*>(pa[g] + static_cast<size_t>(it + u) * 64);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) step(qb[u], qa[u]);
    }
    for (; it < end; ++it) {
        uint4 qa[RG];
        const uint4 qb = *reinterpret_cast<const uint4*>(pb + static_cast<size_t>(it) * 64);
#pragma unroll
        for (int g = 0; g < RG; ++g) qa[g] = *reinterpret_cast<const uint4*>(pa[g] + static_cast<size_t>(it) * 64);
        step(qb, qa);
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) part[wave][g][lane] = acc0[g] + acc1[g];
    __syncthreads();
    if (wave != 0 || col >= N) return;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        v4i sum = part[0][g][lane];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w) sum += part[w][g][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * g + (lane >> 4) * 4 + r;
            if (row < M) {
                const int a = sum[r] >> 8;
                float y = static_cast<float>(a) * sx[g][r];
                y = y * sw;
                Y[static_cast<size_t>(row) * N + col] = y;
                if (WRITE_ACC) acc_out[static_cast<size_t>(row) * N + col] = a;
            }
        }
    }
}

template <int kDecodeWaves, int RG>
void launch_m16(dim3 grid, hipStream_t s, const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                const float* w_scale, int M, int N, int K, float* Y, int32_t* acc_out) {
    if (acc_out)
        hipLaunchKernelGGL((w4a4_gemm_m16<true, kDecodeWaves, RG>), grid, dim3(64 * kDecodeWaves), 0, s, Xq, x_scale,
                           Wq, w_scale, M, N, K, Y, acc_out);
    else
        hipLaunchKernelGGL((w4a4_gemm_m16<false, kDecodeWaves, RG>), grid, dim3(64 * kDecodeWaves), 0, s, Xq,
                           x_scale, Wq, w_scale, M, N, K, Y, acc_out);
}

template <int kDecodeWaves>
void launch_m16_rows(dim3 grid, hipStream_t s, const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                     const float* w_scale, int M, int N, int K, float* Y, int32_t* acc_out) {
    switch ((M + 15) / 16) {
        case 1: launch_m16<kDecodeWaves, 1>(grid, s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out); break;
        case 2: launch_m16<kDecodeWaves, 2>(grid, s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out); break;
        case 3: launch_m16<kDecodeWaves, 3>(grid, s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out); break;
        case 4: launch_m16<kDecodeWaves, 4>(grid, s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out); break;
        case 5:
        case 6: launch_m16<kDecodeWaves, 6>(grid, s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out); break;
        default: launch_m16<kDecodeWaves, 8>(grid, s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out); break;
    }
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                            const float* w_scale, int M, int N, int K, float* Y,
                            int32_t* acc_out, int kernel, hipStream_t s) {
    if (kernel == 3 || kernel == 0) {
        const int slices = w4a4_gemm_fp6_split_slices(M, N, K, kernel == 3);
        if (slices >= 2 || (kernel == 3 && slices == 1))
            return launch_w4a4_gemm_fp6_split(Xq, x_scale, Wq, w_scale, M, N, K, slices, Y, acc_out, s);
        if (kernel == 3) return hipErrorInvalidDevice;
    }
    if (kernel == 2 || (kernel == 0 && w4a4_gemm_fp6_applies(M, N, K)))
        return launch_w4a4_gemm_fp6(Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out, s);
    if (M <= 128 && K % 128 == 0) {
        dim3 grid(static_cast<unsigned>((N + 15) / 16));
        // many column groups (gate/up): two waves each, so that every wave
        // streams a longer K range; few (qkv, o_proj, down): eight waves.
        // Past 64 rows a wide grid leaves this kernel compute- and L2-bound
        // (128 x 24576 x 4096: 73 us against 64 on the FP6 tiles): tiles then.
        const int cus = device_cu_count();
        const bool wide = cus > 0 && static_cast<long long>(grid.x) >= 4LL * cus;
        if (M <= 64 || !wide) {
            if (wide)
                launch_m16_rows<2>(grid, s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out);
            else
                launch_m16_rows<8>(grid, s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out);
            return hipGetLastError();
        }
    }
    if (K % kStepCodes == 0) {
        const long long tiles = static_cast<long long>((N + kT - 1) / kT) * ((M + kT - 1) / kT);
        {
            // 256 x 384 tiles where they fill the last round of workgroups
            // better (qkv_proj: 256 instead of 384 tiles on 256 CUs)
            const int cus = device_cu_count();
            const long long wide = static_cast<long long>(N / kWTN) * (M / kWTM);
            auto fill = [&](long long t) { return static_cast<double>(t) / (((t + cus - 1) / cus) * cus); };
            if (cus > 0 && N % kWTN == 0 && M % kWTM == 0 && fill(wide) > fill(tiles) + 0.05) {
                if (acc_out)
                    hipLaunchKernelGGL((w4a4_gemm_wide<true>), dim3(static_cast<unsigned>(wide)), dim3(kWThreads), 0,
                                       s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out);
                else
                    hipLaunchKernelGGL((w4a4_gemm_wide<false>), dim3(static_cast<unsigned>(wide)), dim3(kWThreads), 0,
                                       s, Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out);
                return hipGetLastError();
            }
        }
        dim3 grid(static_cast<unsigned>(tiles));
        if (acc_out)
            hipLaunchKernelGGL((w4a4_gemm_256<true>), grid, dim3(kGemmThreads), 0, s, Xq, x_scale,
                               Wq, w_scale, M, N, K, Y, acc_out);
        else
            hipLaunchKernelGGL((w4a4_gemm_256<false>), grid, dim3(kGemmThreads), 0, s, Xq, x_scale,
                               Wq, w_scale, M, N, K, Y, acc_out);
        return hipGetLastError();
    }
    // K a multiple of 64 but not of 128: 128 x 128 tiles, 64-code steps
    const long long tiles = static_cast<long long>((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM);
    dim3 grid(static_cast<unsigned>(tiles));
    if (acc_out)
        hipLaunchKernelGGL((w4a4_gemm_basic<true>), grid, dim3(256), 0, s, Xq, x_scale, Wq,
                           w_scale, M, N, K, Y, acc_out);
    else
        hipLaunchKernelGGL((w4a4_gemm_basic<false>), grid, dim3(256), 0, s, Xq, x_scale, Wq,
                           w_scale, M, N, K, Y, acc_out);
    return hipGetLastError();
}

}  // namespace spin
