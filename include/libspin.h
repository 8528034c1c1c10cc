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

/* Status and dtype travel as plain ints: every int a caller passes is a
   valid argument (an unknown dtype is rejected with SPIN_ERR_UNSUPPORTED,
   spin_status_string names an unknown status), which an enum type would not
   allow in C++. */
typedef int spin_status;
enum {
    SPIN_OK = 0,
    SPIN_ERR_NULL = 1,          /* a required pointer is NULL                      */
    SPIN_ERR_BAD_SHAPE = 2,     /* a size is negative, not a required multiple, or too large */
    SPIN_ERR_MISALIGNED = 3,    /* a tensor pointer is not 16-byte aligned         */
    SPIN_ERR_UNSUPPORTED = 4,   /* unsupported Hadamard order, dtype or flag value */
    SPIN_ERR_HIP = 5            /* the HIP runtime reported an error               */
};

typedef int spin_dtype;
enum { SPIN_F32 = 0, SPIN_F16 = 1 };

/* Largest row length spin_fwht_quant accepts. */
#define SPIN_FWHT_MAX_K 32768
/* Most rows one spin_fwht_quant (and _f6, _gemm) call takes, and most
   (token, head) vectors one spin_kv_quant call takes: each kernel launch has
   fewer than 2^32 work-items in its one grid dimension, and these kernels
   give a row 256 of them (rounded up to 256 rows where rows are placed per
   XCD), a workgroup of 256 to 32 KV vectors. */
#define SPIN_FWHT_MAX_M ((1 << 24) - 256)
#define SPIN_KV_MAX_VECTORS (((1LL << 24) - 1) * 32)
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
 * codes.  Requirements: 0 <= M <= SPIN_FWHT_MAX_M, 0 < K <= SPIN_FWHT_MAX_K,
 * K % 32 == 0.
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

/* Kernel families for spin_w4a4_gemm_ex. */
#define SPIN_GEMM_AUTO 0   /* the choice spin_w4a4_gemm makes */
#define SPIN_GEMM_INT8 1   /* codes widened to int8, int8 matrix cores, int32 accumulation */
#define SPIN_GEMM_FP6 2    /* codes as FP6 E2M3 (u = q + 8, exact), FP6 matrix cores */
#define SPIN_GEMM_FP6_SPLITK 3   /* the FP6 tiles with K split into slices; see below */
/* K range of the FP6 kernel: its float32 accumulator of products u_a * u_b <= 225
   is exact while 225 K < 2^24 (K < 74566; the bound stops at the power of two
   below), and its pipeline needs two steps of 128 codes. */
#define SPIN_GEMM_FP6_MIN_K 256
#define SPIN_GEMM_FP6_MAX_K 65536

/*
 * spin_w4a4_gemm_ex — spin_w4a4_gemm with the kernel family named: the same
 * arguments, outputs and guarantees (every family gives the same bits), for
 * callers that tune the choice for their shapes.  `kernel` is SPIN_GEMM_AUTO,
 * SPIN_GEMM_INT8, SPIN_GEMM_FP6 or SPIN_GEMM_FP6_SPLITK.
 * SPIN_GEMM_FP6_SPLITK (taken by AUTO for 129 or more rows whose 256 x 256
 * tiles leave half the compute units idle, when it predicts a gain) is three
 * launches on `stream`: Y is zeroed, the FP6 tiles of every K slice add their
 * exact int32 partial products into Y read as int32 (atomically), and a last
 * pass turns Y into the dequantized float32 outputs in place (and writes
 * acc_out).  The slice count is chosen from the shape (1 when slicing does not
 * pay).  The integer sum is exact and the epilogue the same, so the bits equal
 * the other families'; between the launches Y holds integers.
 * Errors: SPIN_ERR_UNSUPPORTED for another `kernel` value; with
 * SPIN_GEMM_FP6 or SPIN_GEMM_FP6_SPLITK, SPIN_ERR_BAD_SHAPE unless K % 128 == 0
 * and SPIN_GEMM_FP6_MIN_K <= K <= SPIN_GEMM_FP6_MAX_K; otherwise as
 * spin_w4a4_gemm.
 */
spin_status spin_w4a4_gemm_ex(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                              const float* w_scale, int M, int N, int K, float* Y,
                              int32_t* acc_out, int kernel, void* stream);

/*
 * The FP6 operand layout of activation codes, written by spin_fwht_quant_f6
 * and read by spin_w4a4_gemm_f6 and spin_w4a4_gemm_f6f6 (this library's
 * format, also written by spin_codes_f6; the pages fix no
 * storage): the INT4 codes q of an [M][K] activation matrix, each held as the
 * 6-bit field of u = q + 8 (bits 0..3 = u, bits 4..5 = 0: the FP6 E2M3 value
 * u / 8), ordered for the gfx950 matrix cores.  Row r, code k lies in the
 * 1536-byte region (r / 32) * (K / 64) + k / 64, at byte
 * ((k % 64) / 32) * 768 + (r % 32) * 24 + ((k % 32) / 16) * 12 of it, in field
 * sigma(k % 16) of those 12 bytes read as a 96-bit little-endian number (field
 * p at bits 6p .. 6p + 5), sigma = 0 1 12 2 3 14 4 5 11 6 7 13 8 9 15 10.
 * Rows are rounded up to a multiple of 32; the rows past M are padding that
 * spin_fwht_quant_f6 does not write and that no result depends on (they hold
 * whatever the buffer held).  K % 64 == 0.  1.5 bytes per code.
 */
#define SPIN_F6_BYTES(M, K) ((size_t)(((M) + 31) / 32) * ((size_t)(K) / 64) * 1536)

/* Longest row spin_fwht_quant_f6 quantizes without a rotation (had_n == 1). */
#define SPIN_FWHT_F6_QUANT_MAX_K 16384

/*
 * spin_fwht_quant_f6 — spin_fwht_quant (per-token INT4, after the R4 Hadamard
 * or with no rotation, page "SpinQuant, Reproduced", Q5) with the codes
 * written in the FP6 operand layout above, for spin_w4a4_gemm_f6 and
 * spin_w4a4_gemm_f6f6.
 *
 *   X        [M][K] float16 with K == had_n == 12288 (the down projection's
 *            input, R4 online), or float16 / float32 with had_n == 1 (inputs
 *            whose rotation is folded upstream: qkv_proj, o_proj, gate/up)
 *   Xf6      SPIN_F6_BYTES(M, K) bytes   OUTPUT: the codes spin_fwht_quant
 *            computes for the same arguments, in the FP6 operand layout
 *   x_sum    [M] int32     OUTPUT: sum_k q[m][k]
 *   x_scale  [M] float32   OUTPUT: as spin_fwht_quant
 * Requirements: 0 <= M <= SPIN_FWHT_MAX_M; had_n == 12288: x_dtype ==
 * SPIN_F16, K == 12288; had_n == 1: K % 128 == 0, SPIN_GEMM_FP6_MIN_K <= K <=
 * SPIN_FWHT_F6_QUANT_MAX_K.
 * Errors: SPIN_ERR_NULL, SPIN_ERR_UNSUPPORTED for another had_n or dtype,
 * SPIN_ERR_BAD_SHAPE, SPIN_ERR_MISALIGNED (16-byte alignment).
 */
spin_status spin_fwht_quant_f6(const void* X, spin_dtype x_dtype, int M, int K, int had_n, uint8_t* Xf6,
                               int32_t* x_sum, float* x_scale, void* stream);

/*
 * spin_w4a4_gemm_f6 — spin_w4a4_gemm with the activation codes in the FP6
 * operand layout (abstract: W4A4): Y and acc_out are the same bits
 * spin_w4a4_gemm gives for those codes.
 *
 *   Xf6      SPIN_F6_BYTES(M, K) bytes (from spin_fwht_quant_f6)
 *   x_sum    [M] int32, sum_k q[m][k]   x_scale [M] float32
 *   Wq, w_scale, Y, acc_out   as for spin_w4a4_gemm
 * Requirements: M, N >= 0, K % 128 == 0,
 * SPIN_GEMM_FP6_MIN_K <= K <= SPIN_GEMM_FP6_MAX_K.
 */
spin_status spin_w4a4_gemm_f6(const uint8_t* Xf6, const int32_t* x_sum, const float* x_scale,
                              const uint8_t* Wq, const float* w_scale, int M, int N, int K, float* Y,
                              int32_t* acc_out, void* stream);

/*
 * spin_codes_f6 — packed INT4 codes [N][K/2] (spin_fold_rotation's Wq, or
 * the activation codes of spin_fwht_quant) rewritten in the FP6 operand
 * layout above (row n of the codes as row r of the layout), with the code
 * sum of every row, for spin_w4a4_gemm_f6f6.  Weights are static, so theirs
 * is done once, offline (abstract: W4A4), and the conversion of the weight
 * codes into the matrix cores' operand format leaves the hot path.  Any
 * nibble is accepted (-8 becomes the field of u = 0).
 *
 *   Wq     [N][K/2] uint8    packed codes
 *   Wf6    SPIN_F6_BYTES(N, K) bytes   OUTPUT (padding rows past N unwritten)
 *   w_sum  [N] int32         OUTPUT: sum_k q[n][k]
 * Requirements: N >= 0, K > 0, K % 64 == 0, K <= SPIN_GEMM_MAX_K.
 * Errors: SPIN_ERR_NULL for a null pointer, SPIN_ERR_BAD_SHAPE, and
 * SPIN_ERR_MISALIGNED unless every pointer is 16-byte aligned; N == 0 enqueues
 * nothing.
 */
spin_status spin_codes_f6(const uint8_t* Wq, int N, int K, uint8_t* Wf6, int32_t* w_sum, void* stream);

/*
 * spin_w4a4_gemm_f6f6 — spin_w4a4_gemm with both operands in the FP6 operand
 * layout (activations from spin_fwht_quant_f6, weights from spin_codes_f6):
 * Y and acc_out are the same bits spin_w4a4_gemm gives for those codes.
 *
 *   Xf6, x_sum, x_scale   as for spin_w4a4_gemm_f6
 *   Wf6      SPIN_F6_BYTES(N, K) bytes, w_sum [N] int32 (the weight codes
 *            from spin_codes_f6)
 *   w_scale, Y, acc_out   as for spin_w4a4_gemm
 * Requirements: M, N >= 0, K % 128 == 0,
 * SPIN_GEMM_FP6_MIN_K <= K <= SPIN_GEMM_FP6_MAX_K.
 * Errors: SPIN_ERR_NULL, SPIN_ERR_BAD_SHAPE, SPIN_ERR_MISALIGNED (16-byte
 * alignment of every pointer) as for spin_w4a4_gemm_f6; M == 0 or N == 0
 * enqueues nothing.
 */
spin_status spin_w4a4_gemm_f6f6(const uint8_t* Xf6, const int32_t* x_sum, const float* x_scale,
                                const uint8_t* Wf6, const int32_t* w_sum, const float* w_scale, int M, int N,
                                int K, float* Y, int32_t* acc_out, void* stream);

/* 32-bit words of the workspace spin_fwht_quant_gemm takes. */
#define SPIN_FWHT_QUANT_GEMM_WORKSPACE_WORDS 1025

/*
 * spin_fwht_quant_gemm — the down projection's input rotation R4 and its
 * W4A4 product in one launch: spin_fwht_quant followed by spin_w4a4_gemm
 * (page "SpinQuant, Reproduced", Q5: R4 is an online Hadamard right before
 * down_proj; abstract: W4A4).
 *
 *   X          [M][K] float16, K == had_n == 12288 (the MLP width; H_12 (x) H_1024)
 *   Wq, w_scale, N   the folded INT4 weights as for spin_w4a4_gemm
 *   Xq, x_scale      OUTPUT: the codes and scales spin_fwht_quant writes
 *   Y, acc_out       OUTPUT: as spin_w4a4_gemm writes them from those codes
 *   workspace  SPIN_FWHT_QUANT_GEMM_WORKSPACE_WORDS uint32 of device memory,
 *              all zero before the first call; each call leaves it zero.
 * Every output equals, bit for bit, what the two separate calls write.
 * Requirements: x_dtype == SPIN_F16, K == had_n == 12288 (other shapes: the
 * two calls), M, N >= 0; acc_out may be NULL.  Calls that share a workspace
 * must not overlap (calls on one stream do not); the kernel is launched
 * cooperatively (all its workgroups resident at once).
 * Errors: SPIN_ERR_UNSUPPORTED for another dtype or order, SPIN_ERR_BAD_SHAPE,
 * SPIN_ERR_NULL, SPIN_ERR_MISALIGNED as for the two calls; SPIN_ERR_HIP if
 * the device cannot run the cooperative launch.  The wait of a GEMM tile for
 * its rows is bounded (about half a second, or 2^22 polls); it cannot expire
 * while every workgroup is resident, which the cooperative launch ensures,
 * but if it did, that tile's Y would be written as NaN (acc_out INT32_MIN)
 * rather than the kernel hanging.
 */
spin_status spin_fwht_quant_gemm(const void* X, spin_dtype x_dtype, int M, int K, int had_n,
                                 const uint8_t* Wq, const float* w_scale, int N, uint8_t* Xq,
                                 float* x_scale, float* Y, int32_t* acc_out, uint32_t* workspace,
                                 void* stream);

/*
 * spin_fwht_quant_gemm_noalloc — spin_fwht_quant_gemm for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same arguments, outputs and
 * guarantees without the workspace: the flags live in an array of
 * SPIN_FWHT_QUANT_GEMM_WORKSPACE_WORDS words that the library holds in every
 * GPU it runs on until the process ends (its address is looked up on the
 * first call on each device; nothing is allocated).  The array holds the
 * flags of up to 1024 workgroups; the kernel's grid (one workgroup per
 * compute unit) is capped there, so no call needs more.  It is zero before
 * the first call and every call leaves it zero.  All calls on one GPU share
 * it: calls that overlap on one GPU race (calls on one stream do not
 * overlap).  Errors as for spin_fwht_quant_gemm; SPIN_ERR_HIP if the array's
 * address cannot be obtained.
 */
spin_status spin_fwht_quant_gemm_noalloc(const void* X, spin_dtype x_dtype, int M, int K, int had_n,
                                         const uint8_t* Wq, const float* w_scale, int N, uint8_t* Xq,
                                         float* x_scale, float* Y, int32_t* acc_out, void* stream);

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
 * T * H <= SPIN_KV_MAX_VECTORS, D == 128, rotate in {0, 1}.
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

/*
 * spin_kv_qkv — the KV-path step of one attention layer in a single launch
 * (page "SpinQuant, Reproduced", Q5: R3 rotates queries and keys online, so
 * Q . K^T is unchanged, while values carry the folded R2 and are only
 * quantized; abstract: 4-bit KV cache).
 *
 *   Q        [T][Hq][D] float32 / float16, or NULL (no query rotation)
 *   Q_rot    [T][Hq][D] float32, NULL exactly when Q is NULL   OUTPUT:
 *            y = q . H_128 / sqrt(128) per (t, h) vector, not quantized
 *   K, V     [T][Hkv][D], the same dtype as Q; Hq need not equal Hkv
 *            (grouped-query attention)
 *   bits     4: packed INT4 codes, [T][Hkv][D/2] bytes, rules of spin_kv_quant;
 *            8: INT8 codes, [T][Hkv][D] bytes, rules of spin_kv_quant8
 *   K_codes, K_scale   OUTPUT: codes and fp16 scales of K . H_128 / sqrt(128):
 *            the same bytes spin_kv_quant(K, rotate = 1) (spin_kv_quant8 at
 *            bits = 8) writes
 *   K_rot    [T][Hkv][D] float32 or NULL   OUTPUT: the rotated K values
 *   V_codes, V_scale   OUTPUT: codes and fp16 scales of V, not rotated: the
 *            same bytes spin_kv_quant(V, rotate = 0) writes
 * Requirements: T, Hkv >= 0, Hq >= 0 when Q is non-NULL (ignored otherwise),
 * D == 128, bits in {4, 8}; K, V and the four K / V outputs non-NULL.
 * Errors: SPIN_ERR_NULL for a missing pointer or a Q / Q_rot pair with one
 * NULL, SPIN_ERR_UNSUPPORTED for a dtype or bits value outside the above,
 * SPIN_ERR_BAD_SHAPE for a size out of range (2 ceil(T Hkv / 32) + ceil(T Hq / 32)
 * workgroups of 256 above 2^24 - 1, i.e. more than one launch can hold),
 * SPIN_ERR_MISALIGNED as for every call.
 */
spin_status spin_kv_qkv(const void* Q, const void* K, const void* V, spin_dtype x_dtype, int T, int Hq,
                        int Hkv, int D, int bits, float* Q_rot, uint8_t* K_codes, uint16_t* K_scale,
                        float* K_rot, uint8_t* V_codes, uint16_t* V_scale, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* spin_status_string(spin_status s);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int spin_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSPIN_H */
