/*
 * libspin — the online hot path of SpinQuant (arXiv 2405.16406) on AMD
 * Instinct MI355X (gfx950): Hadamard rotations applied online, symmetric INT4
 * quantization of activations / KV vectors, INT4 x INT4 GEMM, and the offline
 * fold of a rotation into a weight.
 *
 * Where each operation comes from (page "SpinQuant, Reproduced"):
 *   - Q1, Q5 "Method 1/2": a pre-norm transformer is invariant to an
 *     orthogonal change of basis of its hidden state; R1 (residual) and R2
 *     (head-wise, value path) are folded into weights; R3 (KV path) and R4
 *     (before down_proj) cannot be folded and run online as Hadamards.
 *   - abstract (all pages): weights, activations and KV cache are 4-bit.
 * The pages fix no interface, granularity, rounding or storage; the choices
 * below (per-token / per-channel / per-(token, head) absmax / 7 scales,
 * round-half-even, clamp to +-7, nibble packing) are this library's reading.
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers to row-major, contiguous memory,
 *     allocated and freed by the caller; the library never allocates, frees
 *     or keeps them.  Every tensor pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls validate their arguments on the host, enqueue kernels on `stream`
 *     and return without synchronising; device faults surface at the caller's
 *     next synchronisation.
 *   - Validation failures return a non-zero spin_status and enqueue nothing,
 *     so no output is written.  SPIN_ERR_HIP means the HIP runtime rejected a
 *     launch; outputs are then undefined.
 *   - Empty problems (M, N, T or H equal to 0) are valid and enqueue nothing.
 *   - The library holds no state; calls are re-entrant and thread-safe.
 *   - INT4 codes are two's-complement nibbles in [-7, 7] (-8 never occurs);
 *     byte j of a packed row holds code 2j in bits 0..3 and code 2j+1 in bits
 *     4..7.
 *   - Hadamard orders ("had_n"): 1 (no rotation), 2^k for 1 <= k <= 14, and
 *     12 * 2^k for 0 <= k <= 10.  H_{2^k} is Sylvester's matrix in natural
 *     order, H[i][j] = (-1)^popcount(i & j).  H_12 is Paley's first
 *     construction over GF(11): with chi the quadratic character mod 11,
 *     Q[a][b] = chi(b - a) and H_12 = I + [[0, 1^T], [-1, Q]] (row/column 0
 *     the border).  H_{12 * 2^k} = H_12 (x) H_{2^k}, element index a*2^k + b.
 *     The rotation applied is the row-vector product y = x . H_n / sqrt(n),
 *     block-diagonally along a row longer than n.
 */
#ifndef LIBSPIN_H
#define LIBSPIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPIN_OK = 0,
    SPIN_ERR_NULL = 1,          /* a required pointer is NULL                      */
    SPIN_ERR_BAD_SHAPE = 2,     /* a size is negative, not a required multiple, or too large */
    SPIN_ERR_MISALIGNED = 3,    /* a tensor pointer is not 16-byte aligned         */
    SPIN_ERR_UNSUPPORTED = 4,   /* unsupported Hadamard order, dtype or flag value */
    SPIN_ERR_HIP = 5            /* the HIP runtime reported an error               */
} spin_status;

typedef enum { SPIN_F32 = 0, SPIN_F16 = 1 } spin_dtype;

/* Largest row length spin_fwht_quant accepts. */
#define SPIN_FWHT_MAX_K 32768
/* Largest K spin_w4a4_gemm accepts: 49 * K * 256 must stay below 2^31
   (the kernel accumulates codes scaled by 16 on each side in int32). */
#define SPIN_GEMM_MAX_K 171136

/*
 * spin_fold_rotation — offline fold of a rotation into a weight, then
 * per-output-channel INT4 (page "SpinQuant, Reproduced", Q5: R1/R2 are merged
 * into adjacent weights and are free at runtime; R4's inverse is merged into
 * down_proj).
 *
 *   W       [K][N] float32   input features x output features
 *   R       [r_block][r_block] float32, or NULL for the library Hadamard
 *           H_{r_block} / sqrt(r_block) (r_block must then be a Hadamard order)
 *   W_rot   [K][N] float32   OUTPUT: W' = blockdiag(R, ..., R)^T W  (required;
 *           it is both the result and the buffer the quantizer reads)
 *   Wq      [N][K/2] uint8   OUTPUT: codes of column n of W', packed
 *   w_scale [N] float32      OUTPUT: fl32(max_k |W'[k][n]| / 7)
 * Codes are clamp(rne(fl32(W'[k][n] / w_scale[n])), -7, 7); a column of zeros
 * gets scale 0 and zero codes.
 * Requirements: K > 0, K % 64 == 0, K % r_block == 0, N >= 0, r_block >= 1.
 * W' accumulates in float32; it is within 1e-5 (relative, per column) of the
 * float64 product.
 */
spin_status spin_fold_rotation(const float* W, int K, int N, const float* R, int r_block,
                               float* W_rot, uint8_t* Wq, float* w_scale, void* stream);

/*
 * spin_fwht_quant — online Hadamard + per-token INT4 of activations (page
 * "SpinQuant, Reproduced", Q5: R4 before down_proj is applied online as a
 * Hadamard over the MLP width; abstract: 4-bit activations).
 *
 *   X        [M][K] float32 (x_dtype SPIN_F32) or float16 (SPIN_F16)
 *   had_n    Hadamard order (see above); 1 = quantize only; K % had_n == 0
 *   Xq       [M][K/2] uint8   OUTPUT: packed codes of y
 *   x_scale  [M] float32      OUTPUT: s = fl32(max_k |y[m][k]| / 7)
 *   X_rot    [M][K] float32 or NULL   OUTPUT: exactly the float32 values y
 *            that were quantized
 * y = x . blockdiag(H_n / sqrt(n)) computed in float32 (within 1e-5 relative
 * per row of the exact product); codes are clamp(rne(fl32(y / s)), -7, 7)
 * with the IEEE float32 quotient, bit-exact; a zero row gets s = 0 and zero
 * codes.  Requirements: M >= 0, 0 < K <= SPIN_FWHT_MAX_K, K % 32 == 0.
 */
spin_status spin_fwht_quant(const void* X, spin_dtype x_dtype, int M, int K, int had_n,
                            uint8_t* Xq, float* x_scale, float* X_rot, void* stream);

/*
 * spin_w4a4_gemm — INT4 x INT4 product with per-token and per-channel scales
 * (abstract: W4A4).
 *
 *   Xq       [M][K/2] uint8   packed activation codes (from spin_fwht_quant)
 *   x_scale  [M] float32
 *   Wq       [N][K/2] uint8   packed weight codes, output-channel-major
 *                             (from spin_fold_rotation)
 *   w_scale  [N] float32
 *   Y        [M][N] float32   OUTPUT: fl32(fl32(float(acc) * x_scale[m]) * w_scale[n])
 *   acc_out  [M][N] int32 or NULL   OUTPUT: acc[m][n] = sum_k qx[m][k] * qw[n][k]
 * The integer product is exact (int32 accumulation, bit-exact) for codes in
 * [-7, 7], the range the library produces; any nibble is accepted, and with
 * -8 codes the bound on K that keeps the sum exact is 64/49 times smaller.
 * Requirements: M, N >= 0, K > 0, K % 64 == 0, K <= SPIN_GEMM_MAX_K.
 */
spin_status spin_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                           const float* w_scale, int M, int N, int K, float* Y,
                           int32_t* acc_out, void* stream);

/*
 * spin_kv_quant — head-wise Hadamard (R3) + INT4 KV cache (page "SpinQuant,
 * Reproduced", Q5: R3 in the KV path is an online Hadamard; abstract: 4-bit
 * KV cache).
 *
 *   X       [T][H][D] float32 / float16, D == 128
 *   rotate  1: y = x . H_128 / sqrt(128) per (t, h) vector (K and Q); 0: y = x (V)
 *   codes   [T][H][D/2] uint8 or NULL   OUTPUT: packed codes of y per (t, h)
 *   scale   [T][H] uint16 (IEEE fp16 bits) or NULL   OUTPUT:
 *           s16 = fp16_rne(fl32(max |y| / 7)); codes use float(s16):
 *           clamp(rne(fl32(y / float(s16))), -7, 7), and s16 == 0 gives zeros
 *   X_rot   [T][H][D] float32 or NULL   OUTPUT: the float32 values y
 * codes and scale are both NULL or both non-NULL; when both are NULL, X_rot
 * must be non-NULL (rotate-only, used for Q).  Requirements: T, H >= 0,
 * D == 128, rotate in {0, 1}.
 */
spin_status spin_kv_quant(const void* X, spin_dtype x_dtype, int T, int H, int D, int rotate,
                          uint8_t* codes, uint16_t* scale, float* X_rot, void* stream);

/*
 * The 8-bit-activation variant, W4A8KV8 (page "SpinQuant, Reproduced", Q7
 * lists it among the settings the paper evaluates): activations and KV
 * vectors are quantized to symmetric INT8 with the same rules as above and
 * 127 in place of 7 (s = fl32(max |y| / 127), codes clamp(rne(fl32(y / s)),
 * -127, 127), one signed byte per code, natural order); weights stay INT4.
 */

/* Largest K spin_w4a8_gemm accepts: 127 * 7 * 16 * K must stay below 2^31
   (weight codes are scaled by 16 in the int32 accumulation). */
#define SPIN_GEMM8_MAX_K 150912

/*
 * spin_fwht_quant8 — spin_fwht_quant with per-token INT8 codes.
 *
 *   Xq8      [M][K] int8      OUTPUT: codes of y
 *   x_scale  [M] float32      OUTPUT: s = fl32(max_k |y[m][k]| / 127)
 * Every other argument, requirement and guarantee as for spin_fwht_quant.
 */
spin_status spin_fwht_quant8(const void* X, spin_dtype x_dtype, int M, int K, int had_n,
                             int8_t* Xq8, float* x_scale, float* X_rot, void* stream);

/*
 * spin_w4a8_gemm — INT8 activations x INT4 weights (W4A8).
 *
 *   Xq8      [M][K] int8      activation codes (from spin_fwht_quant8)
 *   x_scale  [M] float32
 *   Wq       [N][K/2] uint8   packed weight codes (from spin_fold_rotation)
 *   w_scale  [N] float32
 *   Y, acc_out as for spin_w4a4_gemm; the integer product is exact for
 *   activation codes in [-127, 127] and weight codes in [-7, 7] (the ranges
 *   the library produces).
 * Requirements: M, N >= 0, K > 0, K % 128 == 0, K <= SPIN_GEMM8_MAX_K.
 */
spin_status spin_w4a8_gemm(const int8_t* Xq8, const float* x_scale, const uint8_t* Wq,
                           const float* w_scale, int M, int N, int K, float* Y,
                           int32_t* acc_out, void* stream);

/*
 * spin_kv_quant8 — spin_kv_quant with INT8 KV codes (KV8).
 *
 *   codes   [T][H][D] int8 or NULL   OUTPUT: codes of y per (t, h)
 *   scale   [T][H] uint16 (fp16 bits) or NULL   OUTPUT:
 *           s16 = fp16_rne(fl32(max |y| / 127)); codes
 *           clamp(rne(fl32(y / float(s16))), -127, 127), s16 == 0 gives zeros
 * Every other argument, requirement and guarantee as for spin_kv_quant.
 */
spin_status spin_kv_quant8(const void* X, spin_dtype x_dtype, int T, int H, int D, int rotate,
                           int8_t* codes, uint16_t* scale, float* X_rot, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* spin_status_string(spin_status s);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int spin_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSPIN_H */
