/*
 * libspin_probe — machine probes that the benchmark reports beside the
 * published peaks: the sustained dense MFMA rate of the two matrix
 * instructions the hot path issues, the shader clock while the matrix cores
 * are busy, and the streaming read bandwidth of HBM.  Not part of libspin and
 * not used by it.  Calls for callers that measure the machine (bench.py).
 *
 * Conventions as in libspin.h: device pointers allocated by the caller,
 * 16-byte aligned; `stream` is a hipStream_t as void*; arguments are checked on
 * the host and nothing is enqueued when a check fails; the launch is
 * asynchronous.
 */
#ifndef SPIN_PROBE_H
#define SPIN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "libspin.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Dense MFMA loop.  kind 0: v_mfma_i32_32x32x32_i8 (65536 ops each, the INT4
 * GEMM's instruction for K < 8192); kind 1: v_mfma_f32_32x32x16_f16 (32768
 * flops each, the Hadamard stages); kind 2: v_mfma_scale_f32_32x32x64_f8f6f4
 * with FP6 E2M3 operands and block scales 2^3 (131072 ops each, the INT4 GEMM's
 * instruction for long reductions).  `blocks` workgroups of 256 threads (4
 * waves); every wave runs `iters` rounds of four independent MFMAs, i.e.
 * 4 * iters instructions.  `operands`: the data the matrix cores multiply,
 * kinds 0 and 1: 64 lanes x 8 dwords (A in dwords 0-3 of a lane, B in 4-7);
 * kind 2: 64 lanes x 16 dwords (A in dwords 0-5, B in 8-13).  `timing`: 4 int64 per wave (blocks * 4
 * waves): shader-cycle counter at start and end, 100 MHz real-time counter at
 * start and end (the last word may be off by one: it also carries the
 * accumulators so that no chain is optimised away).
 * Errors: SPIN_ERR_NULL, SPIN_ERR_BAD_SHAPE (kind not 0, 1 or 2, blocks or iters
 * out of [1, 2^20] / [1, 2^24]), SPIN_ERR_MISALIGNED, SPIN_ERR_HIP. */
spin_status spin_probe_mfma(int kind, int blocks, int iters, const uint32_t* operands, int64_t* timing,
                            void* stream);

/* Streaming read of `bytes` (a multiple of 16) from `buf` with non-temporal
 * 16-byte loads by `blocks` workgroups of 256 threads in a grid-stride loop.
 * `sink`: one uint32, written only if the data sum hits a fixed improbable
 * value.  Errors: SPIN_ERR_NULL, SPIN_ERR_BAD_SHAPE (bytes 0 or not a multiple
 * of 16, blocks out of [1, 2^20]), SPIN_ERR_MISALIGNED, SPIN_ERR_HIP. */
spin_status spin_probe_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, void* stream);

/* LDS throughput of one compute unit: `blocks` workgroups of 512 threads
 * (eight waves, one workgroup per CU: each holds 96 KB) each fill 64 KB of LDS and then run `iters` rounds of
 * accesses in the patterns of the FP6 GEMM's operand stages.  mode 0: each
 * lane reads 48 bytes per round as six 8-byte loads from 24-byte rows (lane l
 * on row l % 32 of the 768-byte region of k-half l / 32, the MFMA operand
 * reads); mode 1: the same addresses written (the converted fields); mode 2:
 * 48 bytes per round as three 16-byte loads from consecutive addresses.
 * `timing`: 4 int64 per workgroup: shader-cycle counter at start and end,
 * 100 MHz real-time counter at start and end.  `sink`: one uint32, written only
 * if the data meets a fixed improbable value.  Errors: SPIN_ERR_NULL,
 * SPIN_ERR_BAD_SHAPE (mode not 0, 1 or 2, blocks or iters out of [1, 2^20] /
 * [1, 2^24]), SPIN_ERR_MISALIGNED, SPIN_ERR_HIP. */
spin_status spin_probe_lds(int mode, int blocks, int iters, int64_t* timing, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPIN_PROBE_H */
