// Device-side helpers shared by the libspin kernels (gfx950 / CDNA4).
//
// Quantizer (abstract: 4-bit activations, weights, KV cache; the rounding rule
// is this library's reading): code = clamp(rne(fl32(y / s)), -7, 7), s == 0 gives
// 0.  Codes are stored as two's-complement nibbles, two per byte, even element
// in the low nibble.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace spin {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr float kSeven = 7.0f;

// clamp(rne(fl32(y / s)), -7, 7) with the IEEE-correct float32 quotient.
// s == 0 yields 0 (an all-zero group).
__device__ __forceinline__ int quant_exact(float y, float s) {
    if (s == 0.0f) return 0;
    float q = __builtin_rintf(__fdiv_rn(y, s));
    q = __builtin_fminf(__builtin_fmaxf(q, -7.0f), 7.0f);
    return static_cast<int>(q);
}

// The 8-bit variant (W4A8KV8): clamp(rne(fl32(y / s)), -127, 127).
constexpr float kQmax8 = 127.0f;
__device__ __forceinline__ int quant_exact8(float y, float s) {
    if (s == 0.0f) return 0;
    float q = __builtin_rintf(__fdiv_rn(y, s));
    q = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
    return static_cast<int>(q);
}

// fl32(a / d) for d = 7 or 127 without a division instruction sequence:
// q = fl32(a * rd) with rd = fl32(1 / d), the remainder a - d * q is exact in
// one FMA, and q + remainder * rd is rounded once more.  For these two
// divisors the result is the IEEE quotient for every a whose quotient is a
// normal float32 (checked over all 2^23 significands; every step scales
// exactly with a power of two).  A subnormal quotient lies far below the
// smallest fp16 scale, where both values convert to the same fp16 zero.  The
// empty asm keeps the float32 result: without it the compiler may fuse the
// last FMA into a following fp16 conversion, which then rounds the exact sum
// once instead of the float32 quotient.  a must be finite (an infinite a
// gives NaN through the remainder).
constexpr float kRcpSeven = 0x1.24924ap-3f;   // fl32(1 / 7)
constexpr float kRcpQmax8 = 0x1.020408p-7f;   // fl32(1 / 127)
__device__ __forceinline__ float div_by_qmax(float a, float d, float rd) {
    const float q = __fmul_rn(a, rd);
    const float r = __builtin_fmaf(-q, d, a);
    float s = __builtin_fmaf(r, rd, q);
    asm("" : "+v"(s));
    return s;
}

// Four signed byte codes (c[0] lowest) -> one little-endian dword.
__device__ __forceinline__ uint32_t pack4b(const int* c) {
    return (static_cast<uint32_t>(c[0]) & 0xFFu) | ((static_cast<uint32_t>(c[1]) & 0xFFu) << 8) |
           ((static_cast<uint32_t>(c[2]) & 0xFFu) << 16) | ((static_cast<uint32_t>(c[3]) & 0xFFu) << 24);
}

// Eight codes (c[0] lowest) -> one little-endian dword of nibbles.
__device__ __forceinline__ uint32_t pack8(const int* c) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= (static_cast<uint32_t>(c[i]) & 0xFu) << (4 * i);
    return w;
}

__device__ __forceinline__ float load_as_float(const float* p) { return *p; }
__device__ __forceinline__ float load_as_float(const __half* p) { return __half2float(*p); }

// Sign of the Sylvester entry H[i][j] = (-1)^popcount(i & j), as +1 / -1.
__device__ __forceinline__ float sylvester_sign(unsigned i, unsigned j) {
    return (__builtin_popcount(i & j) & 1) ? -1.0f : 1.0f;
}

// Paley-I H_12 over GF(11), row a, as a bit mask of its -1 entries (bit c set
// <=> H12[a][c] == -1).  Row 0 is the +1 border row; column 0 is -1 below it;
// rows 1..11 hold I + Q with Q[a][b] = chi(b - a), residues {1, 3, 4, 5, 9}.
__device__ __forceinline__ unsigned h12_neg_mask(int a) {
    // Written out from the definition, one row per line, bit c = column c.
    constexpr unsigned rows[12] = {
        0x000u,  // + + + + + + + + + + + +
        0xB89u,  // - + + - + + + - - - + -
        0x713u,  // - - + + - + + + - - - +
        0xE25u,  // - + - + + - + + + - - -
        0xC4Bu,  // - - + - + + - + + + - -
        0x897u,  // - - - + - + + - + + + -
        0x12Fu,  // - - - - + - + + - + + +
        0x25Du,  // - + - - - + - + + - + +
        0x4B9u,  // - + + - - - + - + + - +
        0x971u,  // - + + + - - - + - + + -
        0x2E3u,  // - - + + + - - - + - + +
        0x5C5u,  // - + - + + + - - - + - +
    };
    return rows[a];
}

__device__ __forceinline__ float h12_sign(int a, int c) {
    return ((h12_neg_mask(a) >> c) & 1u) ? -1.0f : 1.0f;
}

// Entry (i, j) of the unnormalised library Hadamard of order n = 2^k or 12 * 2^k
// (log2p = k, has12 = n is 12 * 2^k).
__device__ __forceinline__ float hadamard_sign(unsigned i, unsigned j, int log2p, bool has12) {
    const unsigned mask = (1u << log2p) - 1u;
    float s = sylvester_sign(i & mask, j & mask);
    if (has12) s *= h12_sign(static_cast<int>(i >> log2p), static_cast<int>(j >> log2p));
    return s;
}

// Max of a non-negative float over the 16 lanes of each DPP row (every lane
// gets it).  For v >= 0 the float order is the unsigned order of the bit
// patterns, so the reduction runs on the integers: no NaN canonicalisation
// and each level is one v_max_u32 with the DPP operand folded in.
__device__ __forceinline__ float row16_max(float v) {
    unsigned u = __float_as_uint(v);
    u = max(u, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0xB1, 0xF, 0xF, true)));   // lane ^ 1
    u = max(u, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x4E, 0xF, 0xF, true)));   // lane ^ 2
    u = max(u, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x141, 0xF, 0xF, true)));  // lane ^ 7
    u = max(u, static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x140, 0xF, 0xF, true)));  // lane ^ 15
    return __uint_as_float(u);
}

// Block-wide max of non-negative floats over 256 threads (4 waves).  `red`
// is a __shared__ float[4]; the result is returned to every thread.
__device__ __forceinline__ float block_max_256(float v, float* red) {
    v = row16_max(v);
    v = __builtin_fmaxf(v, __shfl_xor(v, 16, 64));
    v = __builtin_fmaxf(v, __shfl_xor(v, 32, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    return __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

}  // namespace spin

namespace spin {

// y = x . H12 (Paley-I, unnormalised) for a row vector of 12, in place.
//
// Every order-12 Hadamard matrix is equivalent to every other under signed
// row and column permutations.  Paley's second construction over GF(5) has
// the block form H' = [[C + I, C - I], [C - I, -C - I]] with C the symmetric
// order-6 conference matrix C = [[0, 1^T], [1, Q5]], Q5[a][b] = chi5(b - a)
// (chi5 = +1 at +-1, -1 at +-2).  Our H12 = P H' S with P, S signed
// permutations (found offline by matching the two matrices row by row), so
// x . H12 = ((x . P) . H') . S.  With u = x . P split as [u1 | u2]:
//   w1 = (u1 + u2) C + (u1 - u2),   w2 = (u1 - u2) C - (u1 + u2),
// and the product of a 6-vector A with C needs, with A' = A[1..5] and
// p_b = A'[b+1] + A'[b-1], S = sum A':  (A C)[0] = S and
// (A C)[1+b] = A[0] - S + A'[b] + 2 p_b.  Folding the + (u1 - u2) and
// - (u1 + u2) terms in gives w1[1+b] = (U0 - S_U) + 2 (p_b(U) + u1[1+b]) and
// w2[1+b] = (V0 - S_V) + 2 (p_b(V) - u2[1+b]).  50 adds / FMAs for 12 outputs
// instead of 132 (paley2_mix below).
// w = u . H' for the Paley-II form H' = [[C + I, C - I], [C - I, -C - I]]
// (see h12_row), in place: 50 adds / FMAs for 12 outputs.
__device__ __forceinline__ void paley2_mix(float (&u)[12]) {
    const float U0 = u[0] + u[6], U1 = u[1] + u[7], U2 = u[2] + u[8], U3 = u[3] + u[9], U4 = u[4] + u[10],
                U5 = u[5] + u[11];
    const float V0 = u[0] - u[6], V1 = u[1] - u[7], V2 = u[2] - u[8], V3 = u[3] - u[9], V4 = u[4] - u[10],
                V5 = u[5] - u[11];
    // p_b over the five non-border entries, indices mod 5
    const float P0 = U2 + U5, P1 = U3 + U1, P2 = U4 + U2, P3 = U5 + U3, P4 = U1 + U4;
    const float SU = P0 + P1 + U4;
    const float EU = U0 - SU;
    const float Q0 = V2 + V5, Q1 = V3 + V1, Q2 = V4 + V2, Q3 = V5 + V3, Q4 = V1 + V4;
    const float SV = Q0 + Q1 + V4;
    const float EV = V0 - SV;
    const float w0 = SU + V0;
    const float w1 = __builtin_fmaf(2.0f, P0 + u[1], EU);
    const float w2 = __builtin_fmaf(2.0f, P1 + u[2], EU);
    const float w3 = __builtin_fmaf(2.0f, P2 + u[3], EU);
    const float w4 = __builtin_fmaf(2.0f, P3 + u[4], EU);
    const float w5 = __builtin_fmaf(2.0f, P4 + u[5], EU);
    const float w6 = SV - U0;
    const float w7 = __builtin_fmaf(2.0f, Q0 - u[7], EV);
    const float w8 = __builtin_fmaf(2.0f, Q1 - u[8], EV);
    const float w9 = __builtin_fmaf(2.0f, Q2 - u[9], EV);
    const float w10 = __builtin_fmaf(2.0f, Q3 - u[10], EV);
    const float w11 = __builtin_fmaf(2.0f, Q4 - u[11], EV);
    u[0] = w0; u[1] = w1; u[2] = w2; u[3] = w3; u[4] = w4; u[5] = w5;
    u[6] = w6; u[7] = w7; u[8] = w8; u[9] = w9; u[10] = w10; u[11] = w11;
}

__device__ __forceinline__ void h12_row(float (&x)[12]) {
    // u = x . P  (input permutation and signs)
    float u[12] = {x[0], x[1], x[2], -x[3], -x[5], -x[7], -x[9], x[4], x[8], -x[6], x[10], -x[11]};
    paley2_mix(u);
    // y = w . S  (output permutation and signs)
    x[0] = u[4];  x[1] = u[11]; x[2] = u[0];  x[3] = u[7]; x[4] = u[5];   x[5] = u[2];
    x[6] = u[1];  x[7] = u[9];  x[8] = -u[6]; x[9] = u[10]; x[10] = u[8]; x[11] = u[3];
}

}  // namespace spin

namespace spin {

// One butterfly level across the 16 lanes of a DPP row, for eight registers:
// r[i] <- r[i] + sgn * r[i] of the partner lane, as a single v_fmac_f32 with a
// DPP source operand.  `sgn` is +1 on the lane of each pair that keeps the sum
// and -1 on the other, which leaves the latter with -(partner - self); the
// sign is carried and removed once at the end.  The partner patterns used are
// quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane ^ 7) and row_mirror (lane ^ 15).  A VALU write of a
// VGPR must be two wait states ahead of a DPP read of it, hence the s_nop.
#define SPIN_DPP_FMAC8(CTRL, r, s)                                                    \
    asm("s_nop 1\n\t"                                                                  \
        "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"            \
        "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                \
        : "+v"((r)[0]), "+v"((r)[1]), "+v"((r)[2]), "+v"((r)[3]), "+v"((r)[4]),        \
          "+v"((r)[5]), "+v"((r)[6]), "+v"((r)[7])                                     \
        : "v"(s))

#define SPIN_DPP_XOR1 "quad_perm:[1,0,3,2]"
#define SPIN_DPP_XOR2 "quad_perm:[2,3,0,1]"
#define SPIN_DPP_XOR7 "row_half_mirror"
#define SPIN_DPP_XOR15 "row_mirror"

// Butterflies along the lane masks 1, 2, 7, 15 realise a Walsh-Hadamard
// transform over the four low lane bits in the coordinates of the dual basis
// phi = {0b0101, 0b0110, 0b1100, 0b1000}: lane i takes sign (-1)^<i, phi_k> at
// level k.  If lane i first holds element g_perm(i) of a 16-point row, lane i
// ends holding element i of its natural-order transform multiplied by
// (-1)^popcount(i & 7).  g_perm is the Gram matrix sum_k phi_k phi_k^T over
// GF(2) acting on the lane bits.
__device__ __forceinline__ int g_perm(int i) {
    const int i0 = i & 1, i1 = (i >> 1) & 1, i2 = (i >> 2) & 1, i3 = (i >> 3) & 1;
    return (i0 ^ i2) | ((i1 ^ i2) << 1) | ((i0 ^ i1 ^ i2 ^ i3) << 2) | (i2 << 3);
}

__device__ __forceinline__ float lane_sign(int l16, int phi) {
    return (__builtin_popcount(l16 & phi) & 1) ? -1.0f : 1.0f;
}

// Four DPP levels over n registers (n a multiple of 8).
template <int NREG>
__device__ __forceinline__ void dpp_wht16(float* r, float s1, float s2, float s3, float s4) {
#pragma unroll
    for (int i = 0; i < NREG; i += 8) SPIN_DPP_FMAC8(SPIN_DPP_XOR1, r + i, s1);
#pragma unroll
    for (int i = 0; i < NREG; i += 8) SPIN_DPP_FMAC8(SPIN_DPP_XOR2, r + i, s2);
#pragma unroll
    for (int i = 0; i < NREG; i += 8) SPIN_DPP_FMAC8(SPIN_DPP_XOR7, r + i, s3);
#pragma unroll
    for (int i = 0; i < NREG; i += 8) SPIN_DPP_FMAC8(SPIN_DPP_XOR15, r + i, s4);
}

// Fast quantizer for a row whose scale s is in the normal range.  With
// cr = norm / s to within two float32 roundings (or three where 1/s comes
// from v_rcp_f32, accurate to one ulp), signed per element as needed, the fused
// f = fma(z, cr, kQuantMagic) lands y/s + 1/2 on a grid of 2^-16 in the low
// mantissa bits: bits 16..19 hold the nibble of floor(y/s + 1/2) and bits
// 0..15 the fraction, offset by one unit so that an exact tie reads 1.
// Whenever the fraction is within one unit of a tie (bits 0..15 < 3) the
// caller recomputes the code with the exact IEEE quotient.  The fast estimate
// is within a few float32 ulps (< 2^-18 absolute) of fl32(y / s), so outside
// that window both round to the same integer.
constexpr float kQuantMagic = 192.5f + 0x1p-16f;

__device__ __forceinline__ bool near_tie(uint32_t fbits) { return (fbits & 0xFFFFu) < 3u; }

// 8-bit codes: f = fma(z, cr, kQuant8Magic) lands y/s + 1/2 on a grid of 2^-14
// (f in [512, 1024) for |y/s| <= 127.5): bits 14..21 hold the two's-complement
// byte of floor(y/s + 1/2), bits 0..13 the fraction, offset by two units so
// that an exact tie reads 2.  The estimate of y/s is within ~0.8 units of
// fl32(y / s) at |y/s| <= 127.5 (float32 roundings of relative size 2^-24 at
// magnitude < 2^7, and 2^-23 where 1/s comes from v_rcp_f32, which is
// accurate to one ulp), plus half a unit from rounding f itself; a fraction
// below 5 units (two below a tie to three above) sends the code to the exact
// IEEE quotient.
constexpr float kQuant8Magic = 768.5f + 0x1p-13f;

__device__ __forceinline__ bool near_tie8(uint32_t fbits) { return (fbits & 0x3FFFu) < 5u; }

// Four 8-bit magic-number results -> one dword of codes (byte k from f[k]).
__device__ __forceinline__ uint32_t pack4_magic8(const uint32_t* f) {
    const uint32_t lo = __builtin_amdgcn_perm(f[1] << 2, f[0] << 2, 0x0c0c0602u);   // f0.b2, f1.b2
    const uint32_t hi = __builtin_amdgcn_perm(f[3] << 2, f[2] << 2, 0x0c0c0602u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// True when any of eight 8-bit magic-number results is near a tie.
__device__ __forceinline__ bool any_near_tie8(const uint32_t* f) {
    const uint32_t m01 = min(f[0] & 0x3FFFu, f[1] & 0x3FFFu), m23 = min(f[2] & 0x3FFFu, f[3] & 0x3FFFu);
    const uint32_t m45 = min(f[4] & 0x3FFFu, f[5] & 0x3FFFu), m67 = min(f[6] & 0x3FFFu, f[7] & 0x3FFFu);
    return min(min(m01, m23), min(m45, m67)) < 5u;
}

// FP6 operand fields.  Sixteen two's-complement nibbles q (two dwords, nibble
// k at bits 4k of a:b) -> sixteen 6-bit fields (three dwords) holding the
// offset codes u = q + 8: nibble k goes to field sigma(k) (bits 6 sigma(k) ..
// + 5 of o[0]:o[1]:o[2]) with sigma = 0 1 12 2 3 14 4 5 11 6 7 13 8 9 15 10,
// u in the field's low four bits and the top two bits zero, so that the field
// is the FP6 E2M3 value u / 8.  u is q with its top bit flipped; the flips
// are not applied to the inputs but to the outputs, where they are bit 3 of
// every field, merged into the masking: per output dword one shift (or funnel
// shift) and two three-input bit operations, (x & M) ^ C and (y & M') ^ that,
// nine instructions in all.
__device__ __forceinline__ void spread16_offset(uint32_t a, uint32_t b, uint32_t* o) {
    // bitop3 table 0x6A: (S0 & S1) ^ S2 (entry index S0 S1 S2, high to low)
    auto and_xor = [](uint32_t x, uint32_t m, uint32_t c) { return __builtin_amdgcn_bitop3_b32(x, m, c, 0x6A); };
    o[0] = and_xor(a << 2, 0xC03C03C0u, and_xor(a, 0x0F00F00Fu, 0x08208208u));
    o[1] = and_xor(__builtin_amdgcn_alignbit(b, a, 30), 0x03C03C03u, and_xor(b, 0xF00F00F0u, 0x82082082u));
    o[2] = and_xor(b << 2, 0x3C03C03Cu, and_xor(a, 0x00F00F00u, 0x20820820u));
}

}  // namespace spin
