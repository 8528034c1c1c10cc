// spin_w4a4_gemm on the gfx950 FP6 matrix cores (abstract: W4A4; per-token
// activation scales and per-output-channel weight scales are this library's
// reading).
//
// The block-scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 multiplies FP6
// operands at twice the int8 MFMA's rate per instruction.  An INT4 code q is
// carried exactly as an FP6 E2M3 value through the offset u = q + 8 in
// [0, 15]: the 6-bit pattern 00uuuu is the E2M3 value u / 8 (exponent field 0
// is subnormal m / 8, exponent field 1 is 1 + m / 8 = (8 + m) / 8, so the
// four low bits read as one unsigned number), and u is the two's-complement
// nibble with its top bit flipped.  With both block scales 2^3 every product
// is u_a u_b, an integer, and the float32 accumulator holds
//     sum_k u_a u_b = sum_k q_a q_b + 8 sum_k q_a + 8 sum_k q_b + 64 K
// exactly while 225 K < 2^24 (K <= 65536 here).  The row sums of the codes
// come from v_dot8_i32_i4 on the packed nibbles, one instruction per eight
// codes, and the epilogue subtracts them, so the integer result is the exact
// dot product of the codes, as the int8 kernels give it.
//
// Conversion: a 16-byte chunk (32 codes of one row) becomes one lane's MFMA
// operand, six dwords holding 32 consecutive 6-bit fields.  Each pair of
// source dwords (16 nibbles) is spread into three dwords with nine shift and
// three-input bit instructions that also flip the top bit of every code
// (spread16_offset); the nibble -> field order
// this gives is the same for both operands, so the dot product over k is
// unchanged.
//
// w4a4_gemm_fp6: 256 x 256 output tile per workgroup of 8 waves (two per
// SIMD), each wave 128 x 64 as 4 x 2 tiles of the 32x32x64 MFMA; a step is 128
// codes (two MFMA k-steps) and ends in the one barrier of the step.
//   * Thread (w, l) owns k-half l / 32 of both k-steps of row 32 w + l % 32
//     of A and of B: four 16-byte chunks per step, loaded from global memory
//     into registers one step before they are converted (lanes l and l + 32
//     read one 32-byte row segment, the two k-steps of a row are adjacent).
//     Each code is converted once for the whole workgroup.
//   * The fields go to a ring of three LDS stages (48 KB each) as regions of
//     32 rows x 24 bytes indexed by (k-step, block of 32 rows, k-half); lane
//     l of a wave reads row l % 32 of the k-half l / 32 region (24-byte rows:
//     the 8-byte accesses of 16 or 32 consecutive rows hit distinct banks).
//     While step s is multiplied from one stage, step s + 1 is complete in
//     the next and step s + 2 is converted into the third, so the operands
//     of the next k-step are read while the current one's MFMAs run: each
//     A operand is reloaded as soon as its second MFMA has issued, and the
//     B operands alternate between two register sets.
//   * Every operand of a k-step is read from its own base register so that
//     the compiler does not pair 8-byte reads of different operands (the
//     pair would then have to be moved into the MFMA's register tuple).
//   * The conversion of step s + 2 is interleaved with the 16 MFMAs of step
//     s (half a chunk after every MFMA pair in program order, the results
//     pinned in place, one scheduling barrier per k-step: a barrier after every
//     pair measured 2% slower), each chunk's fields written as soon as they
//     are complete.
// Rows beyond M or N load the last row; their results are never stored.
// Tiles are ordered XCD-aware as in the int8 kernels.
//
// Measured on MI355X (random codes, K = 12288): a step takes about 3500
// cycles whether 16 or 256 CUs are busy, against 1024 cycles of MFMA work
// per SIMD.  Timing the kernel with parts of the step removed (in a copy):
// without the MFMAs it is no faster (the matrix cores are hidden); without
// the operand reads about 3% faster, with operands that hit in cache 5%,
// without the barrier 13%; without the conversion and the field writes 43%
// faster.  The bound is the conversion pipeline (about 120 VALU instructions
// per wave and step, close to the minimum for this encoding, and the LDS
// writes that follow them), not the matrix cores.  Designs measured slower:
// loads three steps ahead (registers spill), one wave per SIMD with
// 128 x 128 wave tiles (a single wave overlaps neither its ALU work with its
// MFMAs nor LDS latency), 64-code steps (one barrier per 8 MFMAs per wave),
// raw codes staged in LDS by DMA (extra LDS traffic), and 32-byte LDS rows
// (one third more operand bytes).
#pragma once

#include "gemm_common.h"
#include "spin_device.h"

namespace spin {
namespace fp6 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kF6T = 256;
constexpr int kF6Threads = 512;
constexpr int kF6StepCodes = 128;                             // two MFMA k-steps
constexpr int kF6StepBytes = kF6StepCodes / 2;
constexpr int kF6Region = 32 * 24;                            // 32 rows x 24 bytes
constexpr int kF6Blocks = 2 * kF6T / 32;                      // 8 of A, then 8 of B
constexpr int kF6KsBytes = kF6Blocks * 2 * kF6Region;         // one k-step: blocks x k-halves
constexpr int kF6StageBytes = 2 * kF6KsBytes;
constexpr int kF6Scale = 127 + 3;                             // E8M0 block scale 2^3

// Workgroup barrier after this wave's LDS writes have completed; unlike
// __syncthreads it does not wait for the global loads still in flight for
// later steps.  No instruction is scheduled across it: register-only work of
// a later step hoisted above it would wait for that step's loads here.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// One 16-byte chunk of packed codes -> six dwords of FP6 fields (u = q + 8),
// and the sum of its 32 codes added to `sum`.
__device__ __forceinline__ void chunk_to_fp6(uint4 q, uint32_t* o, int& sum) {
    sum = __builtin_amdgcn_sdot8(static_cast<int>(q.x), 0x11111111, sum, false);
    sum = __builtin_amdgcn_sdot8(static_cast<int>(q.y), 0x11111111, sum, false);
    sum = __builtin_amdgcn_sdot8(static_cast<int>(q.z), 0x11111111, sum, false);
    sum = __builtin_amdgcn_sdot8(static_cast<int>(q.w), 0x11111111, sum, false);
    spread16_offset(q.x, q.y, o);
    spread16_offset(q.z, q.w, o + 3);
}

// Keeps three computed dwords where they are in the instruction stream (no
// instruction is emitted): without a use the arithmetic producing them would
// be placed next to the LDS writes that consume them.
__device__ __forceinline__ void pin3(uint32_t* o) { asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2])); }

// A value the compiler cannot relate to any other (no instruction is emitted).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// The epilogue of a wave's 128 x 64 part of a tile: acc = sum u_a u_b ->
// the exact dot product of the codes (minus 8 times the row's and the
// column's code sums and 64 per code), then Y = fl32(fl32(acc * s_x) * s_w),
// or with SPLIT an atomic int32 addition of acc into Y.  Result register r of
// lane l of accumulator (i, j) holds tile row 128 wm + 32 i + 8 (r / 4) +
// 4 (l / 32) + r % 4 and column 64 wn + 32 j + l % 32.  The row and column
// values come from the LDS (`sums_a`, `sums_b`, `sc_a`, `sc_b`, indexed by
// tile row and column); they are read in batches of 16 before any store.
// Tiles inside M and N store without per-element checks, from one address
// per lane and a wave-uniform row offset.
template <bool WRITE_ACC, bool SPLIT>
__device__ __forceinline__ void tile_epilogue(const v16f (&acc)[4][2], const int* sums_a, const int* sums_b,
                                              const float* sc_a, const float* sc_b, int k64, int M, int N, int m0,
                                              int n0, int wm, int wn, int lane, float* __restrict__ Y,
                                              int32_t* __restrict__ acc_out) {
    const int rl = 128 * wm + 4 * (lane >> 5);   // the lane's first tile row
    const int cl = 64 * wn + (lane & 31);        // and column
    int sb[2];
    float sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        sb[j] = sums_b[cl + 32 * j];
        sw[j] = SPLIT ? 0.0f : sc_b[cl + 32 * j];
    }
    const size_t lane_off = static_cast<size_t>(m0 + rl) * N + (n0 + cl);
    auto emit = [&](auto checked) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int sa[16];
            float sx[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rt = rl + 32 * i + 8 * (r >> 2) + (r & 3);
                sa[r] = sums_a[rt];
                sx[r] = SPLIT ? 0.0f : sc_a[rt];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ro = 32 * i + 8 * (r >> 2) + (r & 3);
                const size_t off = lane_off + static_cast<size_t>(ro) * N;
                const bool row_ok = m0 + rl + ro < M;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int a = static_cast<int>(acc[i][j][r]) - 8 * (sa[r] + sb[j]) - k64;
                    const bool ok = !decltype(checked)::value || (row_ok && n0 + cl + 32 * j < N);
                    if (SPLIT) {
                        if (ok) atomicAdd(reinterpret_cast<int*>(Y) + off + 32 * j, a);
                    } else {
                        float y = static_cast<float>(a) * sx[r];
                        y = y * sw[j];
                        if (ok) {
                            Y[off + 32 * j] = y;
                            if (WRITE_ACC) acc_out[off + 32 * j] = a;
                        }
                    }
                }
            }
        }
    };
    if (m0 + kF6T <= M && n0 + kF6T <= N)
        emit(std::false_type{});
    else
        emit(std::true_type{});
}

// One 256 x 256 output tile (tm, tn) by the workgroup of kF6Threads threads,
// on `lds` (three stages of kF6StageBytes, 1024-byte aligned).  Every thread of
// the workgroup calls it; it returns once the tile's stores are issued, with
// the first stage still holding the tile's code sums (read by the epilogue).
// By default the whole reduction; with nsteps >= 0 only the 128-code steps
// s0 .. s0 + nsteps - 1 (at least two).  SPLIT: the exact int32 dot products of
// that range (their own code-sum corrections applied) are added atomically
// into Y read as int32, for a later dequantizing pass; x_scale, w_scale and
// acc_out are not used.
template <bool WRITE_ACC, bool SPLIT = false>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ Xq, const float* __restrict__ x_scale,
                                          const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale,
                                          int M, int N, int K, float* __restrict__ Y,
                                          int32_t* __restrict__ acc_out, int tm, int tn, uint8_t* lds,
                                          int s0 = 0, int nsteps = -1) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m0 = tm * kF6T, n0 = tn * kF6T;
    const size_t rowBytes = static_cast<size_t>(K) / 2;
    const int steps = nsteps >= 0 ? nsteps : K / kF6StepCodes;

    // Thread (w, l) converts k-half h = l / 32 of both k-steps of row
    // 32 w + l % 32 of A and of B in every step: four 16-byte chunks, loaded
    // one step ahead into registers (lanes l and l + 32 read the two halves
    // of one 32-byte row segment, and the two k-steps are adjacent), each
    // becoming the six dwords of one MFMA operand lane in the FP6 stage:
    // region (k-step, block w of A or 8 + w of B, k-half h), row l % 32.
    const int r = 32 * wave + (lane & 31);
    const int h = lane >> 5;
    const uint32_t offA = static_cast<uint32_t>(min(r, M - m0 - 1)) * static_cast<uint32_t>(rowBytes) + 16u * h;
    const uint32_t offB = static_cast<uint32_t>(min(r, N - n0 - 1)) * static_cast<uint32_t>(rowBytes) + 16u * h;
    const uint8_t* baseA = Xq + static_cast<size_t>(m0) * rowBytes + static_cast<size_t>(s0) * kF6StepBytes;
    const uint8_t* baseB = Wq + static_cast<size_t>(n0) * rowBytes + static_cast<size_t>(s0) * kF6StepBytes;
    const uint32_t dstA = (wave * 2 + h) * kF6Region + (lane & 31) * 24;
    const uint32_t dstB = dstA + 8 * 2 * kF6Region;
    int sumA = 0, sumB = 0;

    // operand reads: lane l takes row l % 32, k-half l / 32 of a region; each
    // of the six operands of a k-step has its own base register, so that the
    // compiler does not pair reads of different operands
    const int wm = wave >> 2, wn = wave & 3;
    const uint32_t fr = lds_addr(lds) + (lane >> 5) * kF6Region + (lane & 31) * 24;
    uint32_t fbase[6];
#pragma unroll
    for (int i = 0; i < 4; ++i) fbase[i] = opaque(fr + (4 * wm + i) * 2 * kF6Region);
#pragma unroll
    for (int j = 0; j < 2; ++j) fbase[4 + j] = opaque(fr + (8 + 2 * wn + j) * 2 * kF6Region);

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    typedef const __attribute__((address_space(3))) uint64_t* lds_u64;
    auto frag = [&](int off, int f) {
        const lds_u64 a = reinterpret_cast<lds_u64>(static_cast<uintptr_t>(fbase[f] + off));
        const uint64_t x = a[0], y = a[1], z = a[2];
        const int u = __builtin_nondeterministic_value(0);   // the operand reads six dwords
        return v8i{static_cast<int>(x), static_cast<int>(x >> 32), static_cast<int>(y), static_cast<int>(y >> 32),
                   static_cast<int>(z), static_cast<int>(z >> 32), u, u};
    };
    auto load = [&](int step, uint4* p) {
        const size_t o = static_cast<size_t>(step) * kF6StepBytes;
        p[0] = *reinterpret_cast<const uint4*>(baseA + o + offA);
        p[1] = *reinterpret_cast<const uint4*>(baseA + o + 32 + offA);
        p[2] = *reinterpret_cast<const uint4*>(baseB + o + offB);
        p[3] = *reinterpret_cast<const uint4*>(baseB + o + 32 + offB);
    };
    auto put = [&](uint8_t* d, const uint32_t* o) {
        uint2* q = reinterpret_cast<uint2*>(d);
        q[0] = make_uint2(o[0], o[1]);
        q[1] = make_uint2(o[2], o[3]);
        q[2] = make_uint2(o[4], o[5]);
    };
    auto convert = [&](int stage, const uint4* p) {
        uint8_t* st = lds + stage * kF6StageBytes;
        uint32_t o[6];
        chunk_to_fp6(p[0], o, sumA);
        put(st + dstA, o);
        chunk_to_fp6(p[1], o, sumA);
        put(st + kF6KsBytes + dstA, o);
        chunk_to_fp6(p[2], o, sumB);
        put(st + dstB, o);
        chunk_to_fp6(p[3], o, sumB);
        put(st + kF6KsBytes + dstB, o);
    };
    // Operands in registers: the four A operands of the k-step being
    // multiplied (each reloaded with the next k-step's as soon as its second
    // MFMA has issued) and two sets of the two B operands (k-steps alternate).
    v8i fa[4], fbx[2], fby[2];
    auto read_a = [&](uint32_t off) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = frag(off, i);
    };
    // Half of chunk c's conversion (sum of eight codes, three dwords of fields)
    auto conv_half = [&](const uint4* p, int c, int half, uint32_t* o) {
        const uint4 q = p[c];
        int& sum = c < 2 ? sumA : sumB;
        const uint32_t a = half ? q.z : q.x, b = half ? q.w : q.y;
        sum = __builtin_amdgcn_sdot8(static_cast<int>(a), 0x11111111, sum, false);
        sum = __builtin_amdgcn_sdot8(static_cast<int>(b), 0x11111111, sum, false);
        spread16_offset(a, b, o + 3 * half);
        pin3(o + 3 * half);
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // chunk c of a step: A k-step 0, A k-step 1, B k-step 0, B k-step 1
    auto chunk_dst = [&](uint32_t stage_off, int c) {
        return lds + stage_off + (c & 1) * kF6KsBytes + (c < 2 ? dstA : dstB);
    };
    // One step s: the MFMAs of its two k-steps from stage `cur` (the first
    // k-step's operands already in registers), with
    //   * the second k-step's operands read while the first's MFMAs run, and
    //     the next step's first k-step read (stage `nxt`, complete since the
    //     previous barrier) while the second's run;
    //   * CONV: the conversion of step s + 2 (registers p_conv) into stage
    //     `dst`, interleaved with the MFMAs, and the loads of step s + 3 into
    //     p_load;
    // then one barrier.  Three stages: while step s is multiplied from one,
    // the next is complete in another and step s + 2 is written to the third.
    auto body = [&](int s, uint32_t cur, uint32_t nxt, uint32_t dst, const uint4* p_conv, uint4* p_load,
                    bool conv, bool prefetch) {
        if (conv) load(min(s + 3, steps - 1), p_load);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8i* fb = ks == 0 ? fbx : fby;        // this k-step's B operands
            v8i* fbn = ks == 0 ? fby : fbx;       // the next k-step's
            const uint32_t noff = ks == 0 ? cur + kF6KsBytes : nxt;   // where the next k-step lies
            const bool more = ks == 0 || prefetch;
            if (more) {
                fbn[0] = frag(noff, 4);
                fbn[1] = frag(noff, 5);
            }
            fence();
            uint32_t o[6];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[0], acc[i][0], 2, 2, 0,
                                                                          kF6Scale, 0, kF6Scale);
                acc[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[1], acc[i][1], 2, 2, 0,
                                                                          kF6Scale, 0, kF6Scale);
                if (more) fa[i] = frag(noff, i);
                if (conv) {
                    const int c = 2 * ks + (i >> 1);
                    conv_half(p_conv, c, i & 1, o);
                    if (i & 1) put(chunk_dst(dst, c), o);
                }
            }
            fence();
        }
        barrier_lds();
    };

    // prologue: steps 0 and 1 converted into stages 0 and 1, step 2 in
    // registers, the operands of step 0's first k-step read
    uint4 P0[4], P1[4];
    load(0, P0);
    load(min(1, steps - 1), P1);
    convert(0, P0);
    load(min(2, steps - 1), P0);
    convert(1, P1);
    barrier_lds();
    fbx[0] = frag(0, 4);
    fbx[1] = frag(0, 5);
    read_a(0);
    // every body starts with no LDS access in flight (each ends in a
    // barrier that waits for them); so does the loop's first, and the first
    // MFMA need not wait for the reads a body issues ahead of it
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)

    // steps 0 .. steps - 3 convert step s + 2; two per iteration so that the
    // register sets are fixed; the stage offsets rotate
    uint32_t cur = 0, nxt = kF6StageBytes, dst = 2 * kF6StageBytes;
    auto rotate = [&] {
        const uint32_t t = cur;
        cur = nxt;
        nxt = dst;
        dst = t;
    };
    int s = 0;
    for (; s + 3 < steps; s += 2) {
        body(s, cur, nxt, dst, P0, P1, true, true);
        rotate();
        body(s + 1, cur, nxt, dst, P1, P0, true, true);
        rotate();
    }
    if (s + 2 < steps) {
        body(s, cur, nxt, dst, P0, P1, true, true);
        rotate();
        ++s;
    }
    // The epilogue's scales, one per thread (x_scale of tile row t for t <
    // 256, w_scale of tile column t - 256 after), requested two steps before
    // they are used: loaded in the epilogue, each store waited for its own.
    float scale = 0.0f;
    if (!SPLIT)
        scale = tid < kF6T ? x_scale[min(m0 + tid, M - 1)] : w_scale[min(n0 + tid - kF6T, N - 1)];
    body(s, cur, nxt, dst, P0, P1, false, true);
    rotate();
    body(s + 1, cur, nxt, dst, P0, P1, false, false);

    // code sums per operand row (A rows at 0..255, B at 256..511): the two
    // halves of a row sit in lanes l and l + 32; they and the scales go
    // through the first stage (every stage is idle after the last step's
    // barrier)
    sumA += __shfl_xor(sumA, 32, 64);
    sumB += __shfl_xor(sumB, 32, 64);
    int* sums = reinterpret_cast<int*>(lds);
    float* scales = reinterpret_cast<float*>(lds) + 2 * kF6T;
    if (h == 0) {
        sums[r] = sumA;
        sums[kF6T + r] = sumB;
    }
    if (!SPLIT) scales[tid] = scale;
    barrier_lds();
    // the accumulators are final here: the last step's MFMAs sunk into the
    // epilogue would keep their operands live and spill them
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(acc[i][j]));

    tile_epilogue<WRITE_ACC, SPLIT>(acc, sums, sums + kF6T, scales, scales + kF6T, 64 * steps * kF6StepCodes, M, N,
                                    m0, n0, wm, wn, lane, Y, acc_out);
}

// ---------------------------------------------------------------------------
// gemm_tile_f6a: the same tile with the activation codes already in the FP6
// operand layout of spin_fwht_quant_f6 (u = q + 8 fields, one 1536-byte
// region per 32 rows and 64-code k-step, a row block's k-steps adjacent) and
// their row sums given.  The A part of a stage is then eight contiguous 3 KB
// pieces that each wave copies global -> LDS with the LDS DMA (no registers,
// no ALU); only the weight codes are converted, and only their sums are
// formed.  Stage layout (both halves alike): [block of 32 rows][k-step]
// [k-half][row][24 bytes], A at 0 and B at kF6F6aHalf.
constexpr int kF6F6aBlock = 2 * 2 * kF6Region;               // 3 KB: two k-steps x two k-halves
constexpr int kF6F6aHalf = 8 * kF6F6aBlock;                  // 24 KB
static_assert(2 * kF6F6aHalf == kF6StageBytes, "same stage size as the nibble-input tile");

template <bool WRITE_ACC>
__device__ __forceinline__ void gemm_tile_f6a(const uint8_t* __restrict__ Xf6, const int32_t* __restrict__ x_sum,
                                              const float* __restrict__ x_scale, const uint8_t* __restrict__ Wq,
                                              const float* __restrict__ w_scale, int M, int N, int K,
                                              float* __restrict__ Y, int32_t* __restrict__ acc_out, int tm, int tn,
                                              uint8_t* lds) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m0 = tm * kF6T, n0 = tn * kF6T;
    const size_t rowBytes = static_cast<size_t>(K) / 2;
    const int steps = K / kF6StepCodes;
    const int ksteps = K / 64;
    const uint32_t lds0 = lds_addr(lds);

    // A: wave w copies row block m0 / 32 + w (the last block for tiles past M)
    const int rb = min(m0 / 32 + wave, (M + 31) / 32 - 1);
    const uint8_t* srcA = Xf6 + static_cast<size_t>(rb) * ksteps * 1536 + lane * 16;
    const uint32_t dmaA = lds0 + wave * kF6F6aBlock;          // wave-uniform
    auto dma = [&](int step, uint32_t stage_off) {
        const uint8_t* p = srcA + static_cast<size_t>(step) * 2 * 1536;
#pragma unroll
        for (int q = 0; q < 3; ++q)
            lds_dma16(p + q * 1024, __builtin_amdgcn_readfirstlane(dmaA + stage_off + q * 1024));
    };
    // B: thread (w, l) converts k-half l / 32 of both k-steps of weight row
    // 32 w + l % 32: two 16-byte chunks per step, loaded one step ahead.
    const int r = 32 * wave + (lane & 31);
    const int h = lane >> 5;
    const uint32_t offB = static_cast<uint32_t>(min(r, N - n0 - 1)) * static_cast<uint32_t>(rowBytes) + 16u * h;
    const uint8_t* baseB = Wq + static_cast<size_t>(n0) * rowBytes;
    const uint32_t dstB = kF6F6aHalf + wave * kF6F6aBlock + h * kF6Region + (lane & 31) * 24;
    int sumB = 0;

    const int wm = wave >> 2, wn = wave & 3;
    const uint32_t fr = lds0 + (lane >> 5) * kF6Region + (lane & 31) * 24;
    uint32_t fbase[6];
#pragma unroll
    for (int i = 0; i < 4; ++i) fbase[i] = opaque(fr + (4 * wm + i) * kF6F6aBlock);
#pragma unroll
    for (int j = 0; j < 2; ++j) fbase[4 + j] = opaque(fr + kF6F6aHalf + (2 * wn + j) * kF6F6aBlock);

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    typedef const __attribute__((address_space(3))) uint64_t* lds_u64;
    auto frag = [&](uint32_t off, int f) {
        const lds_u64 a = reinterpret_cast<lds_u64>(static_cast<uintptr_t>(fbase[f] + off));
        const uint64_t x = a[0], y = a[1], z = a[2];
        const int u = __builtin_nondeterministic_value(0);   // the operand reads six dwords
        return v8i{static_cast<int>(x), static_cast<int>(x >> 32), static_cast<int>(y), static_cast<int>(y >> 32),
                   static_cast<int>(z), static_cast<int>(z >> 32), u, u};
    };
    auto load_b = [&](int step, uint4* p) {
        const size_t o = static_cast<size_t>(step) * kF6StepBytes;
        p[0] = *reinterpret_cast<const uint4*>(baseB + o + offB);
        p[1] = *reinterpret_cast<const uint4*>(baseB + o + 32 + offB);
    };
    auto put = [&](uint8_t* d, const uint32_t* o) {
        uint2* q = reinterpret_cast<uint2*>(d);
        q[0] = make_uint2(o[0], o[1]);
        q[1] = make_uint2(o[2], o[3]);
        q[2] = make_uint2(o[4], o[5]);
    };
    auto convert_b = [&](uint32_t stage_off, const uint4* p) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            uint32_t o[6];
            chunk_to_fp6(p[ks], o, sumB);
            put(lds + stage_off + dstB + ks * 2 * kF6Region, o);
        }
    };
    v8i fa[4], fbx[2], fby[2];
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // One step s, as in gemm_tile, with
    //   * CONV: the weight codes of step s + 2 (registers p_conv) converted
    //     into stage `dst`, half a chunk after the first and third MFMA pairs
    //     of each k-step; before anything else the step waits for all of
    //     p_conv, then copies step s + 2's activation block into `dst` and
    //     loads step s + 3's weight chunks into p_load, in that order, so
    //     that the compiler's waits for those loads never include a copy
    //     issued after them; the copy is waited for before the barrier;
    //   * the operand reads of the next k-step during the current MFMAs.
    auto body = [&](int s, uint32_t cur, uint32_t nxt, uint32_t dst, const uint4* p_conv, uint4* p_load,
                    bool conv, bool prefetch) {
        if (conv) {
            asm volatile("" ::"v"(p_conv[0].x), "v"(p_conv[0].y), "v"(p_conv[0].z), "v"(p_conv[0].w),
                         "v"(p_conv[1].x), "v"(p_conv[1].y), "v"(p_conv[1].z), "v"(p_conv[1].w));
            dma(s + 2, dst);
            load_b(min(s + 3, steps - 1), p_load);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8i* fb = ks == 0 ? fbx : fby;
            v8i* fbn = ks == 0 ? fby : fbx;
            const uint32_t noff = ks == 0 ? cur + kF6Region * 2 : nxt;
            const bool more = ks == 0 || prefetch;
            if (more) {
                fbn[0] = frag(noff, 4);
                fbn[1] = frag(noff, 5);
            }
            fence();
            uint32_t o[6];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[0], acc[i][0], 2, 2, 0,
                                                                          kF6Scale, 0, kF6Scale);
                acc[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[1], acc[i][1], 2, 2, 0,
                                                                          kF6Scale, 0, kF6Scale);
                if (more) fa[i] = frag(noff, i);
                if (conv && (i & 1) == 0) {
                    const int half = i >> 1;
                    const uint4 q = p_conv[ks];
                    const uint32_t a = half ? q.z : q.x, b = half ? q.w : q.y;
                    sumB = __builtin_amdgcn_sdot8(static_cast<int>(a), 0x11111111, sumB, false);
                    sumB = __builtin_amdgcn_sdot8(static_cast<int>(b), 0x11111111, sumB, false);
                    spread16_offset(a, b, o + 3 * half);
                    pin3(o + 3 * half);
                    if (half) put(lds + dst + dstB + ks * 2 * kF6Region, o);
                }
                fence();
            }
        }
        if (conv) SPIN_WAIT_VMCNT(2);   // this step's copies; the two weight loads may stay in flight
        barrier_lds();
    };

    // prologue: steps 0 and 1 into stages 0 and 1, step 2's weights in
    // registers, the operands of step 0's first k-step read
    uint4 P0[2], P1[2];
    dma(0, 0);
    dma(min(1, steps - 1), kF6StageBytes);
    load_b(0, P0);
    load_b(min(1, steps - 1), P1);
    convert_b(0, P0);
    load_b(min(2, steps - 1), P0);
    convert_b(kF6StageBytes, P1);
    SPIN_WAIT_VMCNT(2);            // the copies; step 2's weight loads may stay in flight
    barrier_lds();
    fbx[0] = frag(0, 4);
    fbx[1] = frag(0, 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag(0, i);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): every body starts with no LDS access in flight

    uint32_t cur = 0, nxt = kF6StageBytes, dst = 2 * kF6StageBytes;
    auto rotate = [&] {
        const uint32_t t = cur;
        cur = nxt;
        nxt = dst;
        dst = t;
    };
    int s = 0;
    for (; s + 3 < steps; s += 2) {
        body(s, cur, nxt, dst, P0, P1, true, true);
        rotate();
        body(s + 1, cur, nxt, dst, P1, P0, true, true);
        rotate();
    }
    if (s + 2 < steps) {
        body(s, cur, nxt, dst, P0, P1, true, true);
        rotate();
        ++s;
    }
    // the epilogue's per-row and per-column values, requested two steps
    // before they are used (as in gemm_tile)
    float scale;
    int xsum = 0;
    if (tid < kF6T) {
        scale = x_scale[min(m0 + tid, M - 1)];
        xsum = x_sum[min(m0 + tid, M - 1)];
    } else {
        scale = w_scale[min(n0 + tid - kF6T, N - 1)];
    }
    body(s, cur, nxt, dst, P0, P1, false, true);
    rotate();
    body(s + 1, cur, nxt, dst, P0, P1, false, false);

    // weight-code sums per column (the two halves of a row sit in lanes l and
    // l + 32), the activation sums and the scales, through the first stage,
    // idle after the last barrier: [B sums | A sums | x scales | w scales]
    sumB += __shfl_xor(sumB, 32, 64);
    int* sums = reinterpret_cast<int*>(lds);
    float* scales = reinterpret_cast<float*>(lds) + 2 * kF6T;
    if (h == 0) sums[r] = sumB;
    if (tid < kF6T) sums[kF6T + tid] = xsum;
    scales[tid] = scale;
    barrier_lds();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(acc[i][j]));

    // epilogue as in gemm_tile
    tile_epilogue<WRITE_ACC, false>(acc, sums + kF6T, sums, scales, scales + kF6T, 64 * K, M, N, m0, n0, wm, wn,
                                    lane, Y, acc_out);
}

// ---------------------------------------------------------------------------
// gemm_tile_f6ab: both operands already in the FP6 operand layout (the
// activations from spin_fwht_quant_f6, the weights packed once by
// spin_codes_f6) with their code sums given.  Every part of a stage is then
// a contiguous 3 KB piece per 32-row block that one wave copies global -> LDS
// with the LDS DMA: wave w copies activation block m0 / 32 + w and weight
// block n0 / 32 + w (the last block for tiles past M or N), six 1 KB copies
// per step and no conversion at all.  Stage layout as in gemm_tile_f6a.
template <bool WRITE_ACC>
__device__ __forceinline__ void gemm_tile_f6ab(const uint8_t* __restrict__ Xf6, const int32_t* __restrict__ x_sum,
                                               const float* __restrict__ x_scale, const uint8_t* __restrict__ Wf6,
                                               const int32_t* __restrict__ w_sum, const float* __restrict__ w_scale,
                                               int M, int N, int K, float* __restrict__ Y,
                                               int32_t* __restrict__ acc_out, int tm, int tn, uint8_t* lds) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m0 = tm * kF6T, n0 = tn * kF6T;
    const int steps = K / kF6StepCodes;
    const int ksteps = K / 64;
    const uint32_t lds0 = lds_addr(lds);

    const int rba = min(m0 / 32 + wave, (M + 31) / 32 - 1);
    const int rbb = min(n0 / 32 + wave, (N + 31) / 32 - 1);
    const uint8_t* srcA = Xf6 + static_cast<size_t>(rba) * ksteps * 1536 + lane * 16;
    const uint8_t* srcB = Wf6 + static_cast<size_t>(rbb) * ksteps * 1536 + lane * 16;
    const uint32_t dmaA = lds0 + wave * kF6F6aBlock;          // wave-uniform
    const uint32_t dmaB = dmaA + kF6F6aHalf;
    auto dma = [&](int step, uint32_t stage_off) {
        const size_t o = static_cast<size_t>(step) * 2 * 1536;
#pragma unroll
        for (int q = 0; q < 3; ++q)
            lds_dma16(srcA + o + q * 1024, __builtin_amdgcn_readfirstlane(dmaA + stage_off + q * 1024));
#pragma unroll
        for (int q = 0; q < 3; ++q)
            lds_dma16(srcB + o + q * 1024, __builtin_amdgcn_readfirstlane(dmaB + stage_off + q * 1024));
    };

    const int wm = wave >> 2, wn = wave & 3;
    const uint32_t fr = lds0 + (lane >> 5) * kF6Region + (lane & 31) * 24;
    uint32_t fbase[6];
#pragma unroll
    for (int i = 0; i < 4; ++i) fbase[i] = opaque(fr + (4 * wm + i) * kF6F6aBlock);
#pragma unroll
    for (int j = 0; j < 2; ++j) fbase[4 + j] = opaque(fr + kF6F6aHalf + (2 * wn + j) * kF6F6aBlock);

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    typedef const __attribute__((address_space(3))) uint64_t* lds_u64;
    auto frag = [&](uint32_t off, int f) {
        const lds_u64 a = reinterpret_cast<lds_u64>(static_cast<uintptr_t>(fbase[f] + off));
        const uint64_t x = a[0], y = a[1], z = a[2];
        const int u = __builtin_nondeterministic_value(0);   // the operand reads six dwords
        return v8i{static_cast<int>(x), static_cast<int>(x >> 32), static_cast<int>(y), static_cast<int>(y >> 32),
                   static_cast<int>(z), static_cast<int>(z >> 32), u, u};
    };
    v8i fa[4], fbx[2], fby[2];
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // One step s: the copies of step s + 2 into stage `dst` issued first, the
    // MFMAs of both k-steps with the next k-step's operands read during the
    // current one's, the copies waited for, one barrier.
    auto body = [&](uint32_t cur, uint32_t nxt, uint32_t dst, int copy_step, bool prefetch) {
        if (copy_step >= 0) dma(copy_step, dst);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8i* fb = ks == 0 ? fbx : fby;
            v8i* fbn = ks == 0 ? fby : fbx;
            const uint32_t noff = ks == 0 ? cur + kF6Region * 2 : nxt;
            const bool more = ks == 0 || prefetch;
            if (more) {
                fbn[0] = frag(noff, 4);
                fbn[1] = frag(noff, 5);
            }
            fence();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[0], acc[i][0], 2, 2, 0,
                                                                          kF6Scale, 0, kF6Scale);
                acc[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[1], acc[i][1], 2, 2, 0,
                                                                          kF6Scale, 0, kF6Scale);
                if (more) fa[i] = frag(noff, i);
                fence();
            }
        }
        if (copy_step >= 0) SPIN_WAIT_VMCNT(0);
        barrier_lds();
    };

    // prologue: steps 0 and 1 into stages 0 and 1, the operands of step 0's
    // first k-step read
    dma(0, 0);
    dma(min(1, steps - 1), kF6StageBytes);
    SPIN_WAIT_VMCNT(0);
    barrier_lds();
    fbx[0] = frag(0, 4);
    fbx[1] = frag(0, 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag(0, i);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): every body starts with no LDS access in flight

    uint32_t cur = 0, nxt = kF6StageBytes, dst = 2 * kF6StageBytes;
    auto rotate = [&] {
        const uint32_t t = cur;
        cur = nxt;
        nxt = dst;
        dst = t;
    };
    int s = 0;
    for (; s + 2 < steps; ++s) {
        body(cur, nxt, dst, s + 2, true);
        rotate();
    }
    // the epilogue's per-row and per-column values (as in gemm_tile)
    float scale;
    int sum;
    if (tid < kF6T) {
        scale = x_scale[min(m0 + tid, M - 1)];
        sum = x_sum[min(m0 + tid, M - 1)];
    } else {
        scale = w_scale[min(n0 + tid - kF6T, N - 1)];
        sum = w_sum[min(n0 + tid - kF6T, N - 1)];
    }
    body(cur, nxt, dst, -1, true);
    rotate();
    body(cur, nxt, dst, -1, false);

    // [A sums | B sums | x scales | w scales] through the first stage, idle
    // after the last barrier
    int* sums = reinterpret_cast<int*>(lds);
    float* scales = reinterpret_cast<float*>(lds) + 2 * kF6T;
    sums[tid] = sum;
    scales[tid] = scale;
    barrier_lds();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(acc[i][j]));
    tile_epilogue<WRITE_ACC, false>(acc, sums, sums + kF6T, scales, scales + kF6T, 64 * K, M, N, m0, n0, wm, wn,
                                    lane, Y, acc_out);
}

}  // namespace fp6
}  // namespace spin
