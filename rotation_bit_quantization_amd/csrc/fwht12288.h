// The R4 / down_proj row transform shared by the fwht_quant kernels and the
// fused down_proj kernel: an fp16 row of 12288 times H12 (x) H1024 / sqrt(12288)
// on the matrix cores, then per-token INT4 / INT8 codes (page "SpinQuant,
// Reproduced", Q5: R4 before down_proj runs online as a Hadamard over the MLP
// width; abstract: 4-bit activations).  Every function is inline.
#pragma once

#include "spin_device.h"

namespace spin {


// ---------------------------------------------------------------------------
// Quantizer epilogue shared by quant_rows and fwht_quant_k12288_mfma.
__device__ __forceinline__ float h2f_lo(uint32_t w) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xFFFFu)));
}
__device__ __forceinline__ float h2f_hi(uint32_t w) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16)));
}

// Eight magic-number results (nibble in bits 16..19) -> one dword of codes.
__device__ __forceinline__ uint32_t pack8_magic(const uint32_t* f) {
    // byte 2 of every result, even elements into `ev`, odd ones into `od`
    const uint32_t ev = __builtin_amdgcn_perm(__builtin_amdgcn_perm(f[6], f[4], 0x0c0c0602u),
                                              __builtin_amdgcn_perm(f[2], f[0], 0x0c0c0602u),
                                              0x05040100u);
    const uint32_t od = __builtin_amdgcn_perm(__builtin_amdgcn_perm(f[7], f[5], 0x0c0c0602u),
                                              __builtin_amdgcn_perm(f[3], f[1], 0x0c0c0602u),
                                              0x05040100u);
    return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
}

// True when any of eight magic-number results is within one unit of a tie.
__device__ __forceinline__ bool any_near_tie(const uint32_t* f) {
    const uint32_t m01 = min(f[0] & 0xFFFFu, f[1] & 0xFFFFu), m23 = min(f[2] & 0xFFFFu, f[3] & 0xFFFFu);
    const uint32_t m45 = min(f[4] & 0xFFFFu, f[5] & 0xFFFFu), m67 = min(f[6] & 0xFFFFu, f[7] & 0xFFFFu);
    return min(min(m01, m23), min(m45, m67)) < 3u;
}

// Codes of eight values z[k] whose true value is y_k = (z[k] * sg[k]) * norm,
// stored at element e (a multiple of 8) of an output row: one dword of
// nibbles (BITS = 4) or two dwords of bytes (BITS = 8).  The fast path (a
// normal, moderate scale s) uses the magic-number estimate with the constant
// c[k] = sg[k] * norm / s and falls back to the exact quotient near a tie.
template <int BITS>
__device__ __forceinline__ void quant8_store(uint8_t* row_out, int e, const float* z, const float* sg,
                                             const float* c, float norm, float s, bool fast) {
    if (BITS == 4) {
        uint32_t word = 0;
        bool exact = !fast;
        if (fast) {
            uint32_t f[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) f[k] = __float_as_uint(__builtin_fmaf(z[k], c[k], kQuantMagic));
            word = pack8_magic(f);
            exact = any_near_tie(f);
        }
        if (exact) {
            int c8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) c8[k] = quant_exact((z[k] * sg[k]) * norm, s);
            word = pack8(c8);
        }
        *reinterpret_cast<uint32_t*>(row_out + e / 2) = word;
    } else {
        uint32_t w0 = 0, w1 = 0;
        bool exact = !fast;
        if (fast) {
            uint32_t f[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) f[k] = __float_as_uint(__builtin_fmaf(z[k], c[k], kQuant8Magic));
            w0 = pack4_magic8(f);
            w1 = pack4_magic8(f + 4);
            exact = any_near_tie8(f);
        }
        if (exact) {
            int c8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) c8[k] = quant_exact8((z[k] * sg[k]) * norm, s);
            w0 = pack4b(c8);
            w1 = pack4b(c8 + 4);
        }
        *reinterpret_cast<uint2*>(row_out + e) = make_uint2(w0, w1);
    }
}

// ---------------------------------------------------------------------------
// fwht_quant_k12288_mfma: the R4 / down_proj case with the two 32-point
// stages of H1024 = H32 (x) H32 on the matrix cores.  On the 32 x 32 view of
// a 1024-block (x[32 i + c] = Xm[i][c]) the Sylvester transform is
// Ym = H32 Xm H32, two products with a +-1 matrix:
//   stage 1  T = Xm H32 with Xm as the A operand straight from the fp16 row
//            (products of fp16 values with +-2^-5 are exact; float32 sums),
//   stage 2  D = T^T H32, with T^T read from stage 1's accumulators, which
//            already sit in A-operand order.  T is float32, so it enters as
//            an fp16 pair hi + lo (hi = fp16(t), lo = fp16(t - hi)), two
//            MFMAs whose sum carries 22 of t's 24 significant bits.
// One wave per row keeps all twelve 1024-blocks in registers, so the H12 mix,
// the absmax and the quantizer run without LDS or a barrier.
//
// Layouts (v_mfma_f32_32x32x16_f16): lane l = 32 h + c supplies row c of A
// (column c of B) with k slots 8 h .. 8 h + 7; accumulator register r of lane
// l holds row 8 (r / 4) + 4 h + r % 4, column c.  Lane l loads x[32 c + 16 h
// .. + 15] (32 contiguous bytes) as k slots (c = 16 h + j, 16 h + 8 + j);
// stage 1's columns are permuted by pi1(8 g + 4 h + s) = 16 h + 4 g + s, so
// that after stage 2 register r of lane l holds element 32 c + 16 h + r:
// sixteen consecutive elements per lane, one 8- or 16-byte store of codes.
//
// The 2^-5 on stage 1 keeps every fp16 hi in range for any finite fp16 row
// (|t| <= 32 * 65504 * 2^-5).  The split loses at most 2^-25 absolute per
// value, which is below 1e-5 of the row's absmax once that absmax (of y) is
// at least 2.  Rows below that (and all-zero rows) are recomputed with stage
// 1 scaled by 2^(m - 5), m = min(20, 29 - E), E the fp16 exponent field of the
// row's largest |x|: that puts max |t| in [2^14, 2^15) for m < 20, and for
// m = 20 every x is a multiple of 2^-24 of magnitude < 2^-6 (the split then
// keeps 22 bits of the row's absmax or is exact).
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

// Sign bits of the +-1 B operands of both stages.  Slot j (bits j0 j1 j2) of
// lane l = 32 h + c holds H32[i][col] with i = 8 (j / 4) + 4 h + j % 4, col = c
// in stage 2 and i = 16 h + j, col = pi1(c) in stage 1 (plus 16, resp. 8, on i
// for the second operand of the pair).  In both cases the parity of i & col
// is the same function of the lane bits c0..c4:
//   (h & c2) ^ (j0 & c0) ^ (j1 & c1) ^ (j2 & c3)   (^ c4 for the second operand)
// sa / sb hold it at bit 15 (even j) and bit 31 (odd j) of dword j / 2.
__device__ __forceinline__ void operand_signs(unsigned lane, u4v& sa, u4v& sb) {
    const unsigned c = lane & 31u, h = lane >> 5;
    const unsigned pair = 0x80008000u;
    const unsigned m1 = (0u - ((c >> 1) & 1u)) & pair;
    const unsigned m3 = (0u - ((c >> 3) & 1u)) & pair;
    const unsigned m4 = (0u - ((c >> 4) & 1u)) & pair;
    const unsigned base = ((0u - (h & (c >> 2) & 1u)) & pair) ^ (c << 31);
    sa = u4v{base, base ^ m1, base ^ m3, base ^ m1 ^ m3};
    sb = sa ^ m4;
}

// Splits eight float32 values t[r0 .. r0 + 7] into fp16 operands hi + lo:
// hi = fp16(t) (packed by the compiler), lo = fp16(t - hi), the difference
// exact in float32, one mixed-precision FMA with -1 per value reading its hi
// half through op_sel.  The compiler does not track the VALU-write -> MFMA-read
// dependency through inline asm, so the block ends with three wait states
// (two are required before an MFMA may read a VGPR that a VALU wrote).  Its
// inputs (the hi words) come from compiler-scheduled conversions that read the
// stage-1 accumulators, so the MFMA-write -> VALU-read wait has already passed.
__device__ __forceinline__ void split8(const f16v& t, int r0, float mone, h8v& hi, h8v& lo) {
    typedef _Float16 h2v __attribute__((ext_vector_type(2)));
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const h2v hp = {static_cast<_Float16>(t[r0 + 2 * p]), static_cast<_Float16>(t[r0 + 2 * p + 1])};
        hw[p] = __builtin_bit_cast(uint32_t, hp);
    }
    asm("v_fma_mixlo_f16 %0, %4, %8, %9 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixlo_f16 %1, %5, %8, %11 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixlo_f16 %2, %6, %8, %13 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixlo_f16 %3, %7, %8, %15 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %4, %8, %10 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %1, %5, %8, %12 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %2, %6, %8, %14 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %3, %7, %8, %16 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "s_nop 2"
        : "=&v"(lw[0]), "=&v"(lw[1]), "=&v"(lw[2]), "=&v"(lw[3])
        : "v"(hw[0]), "v"(hw[1]), "v"(hw[2]), "v"(hw[3]), "s"(mone),
          "v"(t[r0]), "v"(t[r0 + 1]), "v"(t[r0 + 2]), "v"(t[r0 + 3]),
          "v"(t[r0 + 4]), "v"(t[r0 + 5]), "v"(t[r0 + 6]), "v"(t[r0 + 7]));
    hi = __builtin_bit_cast(h8v, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    lo = __builtin_bit_cast(h8v, make_uint4(lw[0], lw[1], lw[2], lw[3]));
}

// y_block (unnormalised, times the stage-1 scale) = x_block . H1024.
__device__ __forceinline__ f16v hadamard1024_mfma(const u4v& x0, const u4v& x1, const h8v& b1a,
                                                  const h8v& b1b, const h8v& b2a, const h8v& b2b,
                                                  float mone) {
    const f16v zero = {};
    f16v t = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, x0), b1a, zero, 0, 0, 0);
    t = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, x1), b1b, t, 0, 0, 0);
    h8v ha, la, hb, lb;
    split8(t, 0, mone, ha, la);
    split8(t, 8, mone, hb, lb);
    f16v u = __builtin_amdgcn_mfma_f32_32x32x16_f16(la, b2a, zero, 0, 0, 0);
    u = __builtin_amdgcn_mfma_f32_32x32x16_f16(lb, b2b, u, 0, 0, 0);
    u = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, b2a, u, 0, 0, 0);
    u = __builtin_amdgcn_mfma_f32_32x32x16_f16(hb, b2b, u, 0, 0, 0);
    return u;
}

// The whole 12288-row: stage 1 (scaled by mag) and stage 2 per 1024-block,
// then the H12 mix across the twelve blocks, in place in u.
// The whole 12288-row: stage 1 (B entries +-mag, mag given by its fp16 bits
// in both halves of magpair) and stage 2 per 1024-block, then the H12 mix
// across the twelve blocks, in place in u.
__device__ __forceinline__ void transform_row12288(const u4v (&raw)[12][2], unsigned magpair, const u4v& sa,
                                                   const u4v& sb, float mone, f16v (&u)[12]) {
    const h8v b1a = __builtin_bit_cast(h8v, sa | magpair), b1b = __builtin_bit_cast(h8v, sb | magpair);
    const h8v b2a = __builtin_bit_cast(h8v, sa | 0x3C003C00u), b2b = __builtin_bit_cast(h8v, sb | 0x3C003C00u);
#pragma unroll
    for (int a = 0; a < 12; ++a) u[a] = hadamard1024_mfma(raw[a][0], raw[a][1], b1a, b1b, b2a, b2b, mone);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float col12[12];
#pragma unroll
        for (int a = 0; a < 12; ++a) col12[a] = u[a][r];
        h12_row(col12);
#pragma unroll
        for (int a = 0; a < 12; ++a) u[a][r] = col12[a];
    }
}

__device__ __forceinline__ float row_absmax(const f16v (&u)[12]) {
    float mx = 0.0f;
#pragma unroll
    for (int a = 0; a < 12; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, __builtin_fabsf(u[a][r]));
    return mx;
}

__device__ __forceinline__ float wave_max64(float v) {
    v = row16_max(v);
    v = __builtin_fmaxf(v, __shfl_xor(v, 16, 64));
    return __builtin_fmaxf(v, __shfl_xor(v, 32, 64));
}

// Sixteen consecutive INT4 codes from the magic-number quantizer (exact
// quotient near a tie or outside the fast range) as two dwords of nibbles.
__device__ __forceinline__ uint2 quant16_nibbles(const f16v& u, float cr, float nrm, float s, bool fast) {
    uint32_t w0 = 0, w1 = 0;
    bool exact = !fast;
    if (fast) {
        uint32_t f[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) f[k] = __float_as_uint(__builtin_fmaf(u[k], cr, kQuantMagic));
        w0 = pack8_magic(f);
        w1 = pack8_magic(f + 8);
        // no short circuit: one branch
        exact = (static_cast<int>(any_near_tie(f)) | static_cast<int>(any_near_tie(f + 8))) != 0;
    }
    if (exact) {
        int c[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) c[k] = quant_exact(u[k] * nrm, s);
        w0 = pack8(c);
        w1 = pack8(c + 8);
    }
    return make_uint2(w0, w1);
}

// Sixteen consecutive codes from the magic-number quantizer (exact quotient
// near a tie or outside the fast range), one store.
template <int BITS>
__device__ __forceinline__ void quant16_store(uint8_t* p, const f16v& u, float cr, float nrm, float s,
                                              bool fast) {
    if (BITS == 4) {
        *reinterpret_cast<uint2*>(p) = quant16_nibbles(u, cr, nrm, s, fast);
    } else {
        uint4 w = make_uint4(0, 0, 0, 0);
        bool exact = !fast;
        if (fast) {
            uint32_t f[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) f[k] = __float_as_uint(__builtin_fmaf(u[k], cr, kQuant8Magic));
            w = make_uint4(pack4_magic8(f), pack4_magic8(f + 4), pack4_magic8(f + 8), pack4_magic8(f + 12));
            exact = (static_cast<int>(any_near_tie8(f)) | static_cast<int>(any_near_tie8(f + 8))) != 0;
        }
        if (exact) {
            int c[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) c[k] = quant_exact8(u[k] * nrm, s);
            w = make_uint4(pack4b(c), pack4b(c + 4), pack4b(c + 8), pack4b(c + 12));
        }
        *reinterpret_cast<uint4*>(p) = w;
    }
}

// The transform of one row by one wave (`lane` = the thread's index in its
// wave): u[a] * nrm are the lane's sixteen values y[1024 a + 32 c + 16 h .. + 15]
// (lane = 32 h + c); returns the row's scale fl32(max |y| / qmax).
template <int BITS>
__device__ __forceinline__ float fwht12288_transform(const __half* __restrict__ X, size_t row, int lane,
                                                     float norm, float mone, f16v (&u)[12], float& nrm) {
    const int h = lane >> 5, c = lane & 31;
    const __half* xr = X + row * 12288 + 32 * c + 16 * h;
    u4v raw[12][2];
#pragma unroll
    for (int a = 0; a < 12; ++a) {  // read once: non-temporal
        raw[a][0] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(xr + a * 1024));
        raw[a][1] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(xr + a * 1024 + 8));
    }
    u4v sa, sb;
    operand_signs(lane, sa, sb);
    nrm = norm * 32.0f;
    transform_row12288(raw, 0x28002800u, sa, sb, mone, u);     // +-2^-5
    float amax = wave_max64(row_absmax(u)) * nrm;       // = max_i fl32(|u_i| * nrm)
    if (!(amax >= 2.0f)) {
        // small (or all-zero) row: reload it and rescale stage 1 from the
        // exact largest |x|
        u4v raw2[12][2];
        uint32_t mb = 0;
#pragma unroll
        for (int a = 0; a < 12; ++a) {
            raw2[a][0] = *reinterpret_cast<const u4v*>(xr + a * 1024);
            raw2[a][1] = *reinterpret_cast<const u4v*>(xr + a * 1024 + 8);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                mb = max(mb, max(raw2[a][0][k] & 0x7FFFu, (raw2[a][0][k] >> 16) & 0x7FFFu));
                mb = max(mb, max(raw2[a][1][k] & 0x7FFFu, (raw2[a][1][k] >> 16) & 0x7FFFu));
            }
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) mb = max(mb, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mb), o, 64)));
        const int m = min(20, 29 - static_cast<int>(mb >> 10));   // m >= -2 for any fp16 row
        nrm = __builtin_ldexpf(norm, 5 - m);
        const unsigned mag = __builtin_bit_cast(unsigned short, static_cast<_Float16>(__builtin_ldexpf(1.0f, m - 5)));
        transform_row12288(raw2, mag * 0x10001u, sa, sb, mone, u);
        amax = wave_max64(row_absmax(u)) * nrm;
    }
    return __fdiv_rn(amax, BITS == 4 ? kSeven : kQmax8);
}

// One row by one wave: codes of row `row` to Xq, its scale to x_scale[row],
// the rotated values to X_rot when WRITE_ROT.
template <int BITS, bool WRITE_ROT>
__device__ __forceinline__ void fwht12288_row(const __half* __restrict__ X, size_t row, int lane, float norm,
                                              float mone, uint8_t* __restrict__ Xq, float* __restrict__ x_scale,
                                              float* __restrict__ X_rot) {
    const int h = lane >> 5, c = lane & 31;
    f16v u[12];
    float nrm;
    const float s = fwht12288_transform<BITS>(X, row, lane, norm, mone, u, nrm);
    if (lane == 0) x_scale[row] = s;
    const bool fast = (s >= 0x1p-100f) && (s <= 0x1p+100f);
    const float cr = fast ? nrm * __fdiv_rn(1.0f, s) : 0.0f;
    const unsigned e0 = 32u * c + 16u * h;
    uint8_t* out = Xq + row * (BITS == 4 ? 6144 : 12288) + e0 * BITS / 8;
#pragma unroll
    for (int a = 0; a < 12; ++a) quant16_store<BITS>(out + a * (1024 * BITS / 8), u[a], cr, nrm, s, fast);
    if (WRITE_ROT) {
        float* yr = X_rot + row * 12288 + e0;
#pragma unroll
        for (int a = 0; a < 12; ++a)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4*>(yr + a * 1024 + 4 * q) =
                    make_float4(u[a][4 * q] * nrm, u[a][4 * q + 1] * nrm, u[a][4 * q + 2] * nrm,
                                u[a][4 * q + 3] * nrm);
    }
}


// One row by one wave with the codes written in the FP6 operand layout of
// spin_fwht_quant_f6 (row block of 32 rows, 64-code k-step: a 1536-byte
// region [k-half][row][24 bytes]; lane 32 h + c holds codes 32 c + 16 h ..
// + 15 of every 1024-block a, i.e. half-group h of k-half c % 2 of k-step
// 16 a + c / 2) and the sum of the row's codes to x_sum[row].
__device__ __forceinline__ void fwht12288_row_f6(const __half* __restrict__ X, size_t row, int lane, float norm,
                                                 float mone, uint8_t* __restrict__ Xf6,
                                                 int32_t* __restrict__ x_sum, float* __restrict__ x_scale) {
    const int h = lane >> 5, c = lane & 31;
    f16v u[12];
    float nrm;
    const float s = fwht12288_transform<4>(X, row, lane, norm, mone, u, nrm);
    if (lane == 0) x_scale[row] = s;
    const bool fast = (s >= 0x1p-100f) && (s <= 0x1p+100f);
    const float cr = fast ? nrm * __fdiv_rn(1.0f, s) : 0.0f;
    uint8_t* out = Xf6 + ((row >> 5) * (12288 / 64) + (c >> 1)) * 1536 + (c & 1) * 768 + (row & 31) * 24 + h * 12;
    int sum = 0;
#pragma unroll
    for (int a = 0; a < 12; ++a) {
        const uint2 w = quant16_nibbles(u[a], cr, nrm, s, fast);
        sum = __builtin_amdgcn_sdot8(static_cast<int>(w.x), 0x11111111, sum, false);
        sum = __builtin_amdgcn_sdot8(static_cast<int>(w.y), 0x11111111, sum, false);
        uint32_t o[3];
        spread16_offset(w.x, w.y, o);
        *reinterpret_cast<uint3*>(out + a * 16 * 1536) = make_uint3(o[0], o[1], o[2]);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m, 64);
    if (lane == 0) x_sum[row] = sum;
}

}  // namespace spin
