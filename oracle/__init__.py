"""CPU oracle for the SpinQuant runtime hot path — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
library is checked against.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does,
and this package imports nothing from the product package.

Source of the method: *SpinQuant: LLM quantization with learned rotations*
(arXiv 2405.16406), as described on the page "SpinQuant, Reproduced"
(romaanj.github.io), sections Q5 "Method 1/2" (where R1..R4 sit, which are
folded and which run online as a Hadamard) and Q3 (kurtosis), plus the abstract
(4-bit weights, activations and KV cache).  The pages fix neither the Hadamard
construction, the quantizer's rounding, granularity and packing, nor the GEMM
accumulation width; the readings taken here are listed per function.

Arithmetic conventions
  * floating point is accumulated in float64 and rounded once to float32;
  * quantizer decisions are taken in float32, exactly as specified
    (IEEE division, round-half-even), because float decides an integer there;
  * integer dot products accumulate in int64 (C routine in ``gemm_int64.c``).

Modules
  hadamard  Sylvester / Paley-I / Kronecker Hadamard matrices, dense rotation
  quant     per-row absmax INT4 / INT8 quantizer, KV fp16-scale quantizer, nibble packing
  fold      W' = B^T W (B block-diagonal rotation) + per-output-channel INT4
  gemm      int64 GEMM on INT4 codes (C) + float32 dequant epilogue
  kv        head-wise Hadamard + per-(token, head) INT4 for the KV path
  stats     kurtosis and orthogonality error
  cayley    Cayley update of an orthogonal matrix (rotation learning, offline)

Parity pins live in ``tests/test_oracle_*.py``; every function here has at
least one pin that does not re-use its own code.
"""

from .hadamard import sylvester, paley12, hadamard, rotate_rows, supported_had_n  # noqa: F401
from .quant import (quantize_rows, quantize_kv_groups, pack_int4, unpack_int4,  # noqa: F401
                    quantize_given_scale)
from .fold import fold_rotation, block_rotation  # noqa: F401
from .gemm import gemm_int_codes, gemm_int_codes_blas, dequant, w4a4_gemm, w4a8_gemm, gemm_rows  # noqa: F401
from .kv import kv_quant, kv_quant8  # noqa: F401
from .stats import kurtosis_per_token, mean_kurtosis, orthogonality_error  # noqa: F401
from .fwht_quant import fwht_quant, fwht_quant8  # noqa: F401
from .cayley import skew_descent, cayley_step  # noqa: F401
