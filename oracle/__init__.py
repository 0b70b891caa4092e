"""CPU oracle for the weight-quantized linear layer (test infrastructure only).

This package is a plain, slow, obviously correct NumPy implementation of what
the GPU library computes.  It exists to check the GPU path and nothing else:
only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import it.  The product path never calls into it, and it shares no code,
tables or helpers with the HIP library.

Precision rules (the same in every module):
  * steps the method performs in fp32 (quantizer min/max/scale/divide/round)
    are emulated with ``np.float32`` arrays, whose ``+ - * /`` are IEEE binary32
    correctly rounded and whose ``np.rint`` rounds half to even;
  * dequantization and the matrix products run in fp64 (integer products in
    int64), so the oracle's own rounding error is far below the tolerance.

Every function is pinned by tests under ``tests/`` (brute force on tiny
inputs, closed forms, invariants, library special cases).  Parity with the
pages' own MLX / Metal / CUDA outputs is unpinned: those implementations are
not available.
"""

from .codecs import (
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    round_to_dtype,
    half_ulp,
    DTYPES,
)
from .affine import (
    affine_quantize,
    affine_pack,
    affine_unpack,
    affine_dequantize,
    affine_forward,
)
from .ternary import ternary_pack, ternary_unpack, ternary_forward
from .int8 import quantize_rows_int8, quantize_rows_int8_clip, row_percentile, int8_matmul_int32, w8a8_forward
from .pergroup import quantize_groups_int8, pergroup_forward
from .w4a8 import pack_weight_int4, unpack_weight_int4, w4a8_forward
from .tolerance import tolerance, compare

__all__ = [
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
    "round_to_dtype",
    "half_ulp",
    "DTYPES",
    "affine_quantize",
    "affine_pack",
    "affine_unpack",
    "affine_dequantize",
    "affine_forward",
    "ternary_pack",
    "ternary_unpack",
    "ternary_forward",
    "quantize_rows_int8",
    "quantize_rows_int8_clip",
    "row_percentile",
    "int8_matmul_int32",
    "w8a8_forward",
    "quantize_groups_int8",
    "pergroup_forward",
    "pack_weight_int4",
    "unpack_weight_int4",
    "w4a8_forward",
    "tolerance",
    "compare",
]
