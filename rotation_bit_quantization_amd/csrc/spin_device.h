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

// Block-wide max of non-negative floats over 256 threads (4 waves).  `red`
// is a __shared__ float[4]; the result is returned to every thread.
__device__ __forceinline__ float block_max_256(float v, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    return r;
}

}  // namespace spin
