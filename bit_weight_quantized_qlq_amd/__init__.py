"""Weight-quantized linear layers on AMD MI355X (gfx950): y = x . dequant(W)^T + b
from packed low-bit codes, through the C ABI of libqlq (include/qlq.h).

Group-wise affine n-bit weights (qlq_pack / qlq_linear_forward), ternary
BitLinear (bitlinear_pack / bitlinear_forward) and per-channel W8A8
(w8a8_linear_forward) with its per-group variant (pergroup_linear_forward),
per-column int4 weights with int8 activations (w4a8_linear_forward), plus
bit-exact helpers.  All computation runs in HIP
kernels; this package only marshals torch tensors into the C ABI.
"""

from .binding import (  # noqa: F401
    QLQError,
    QLQ_OK, QLQ_ERR_INVALID_ARG, QLQ_ERR_UNSUPPORTED, QLQ_ERR_DTYPE, QLQ_ERR_ALIGNMENT,
    QLQ_ERR_WORKSPACE, QLQ_ERR_DATA, QLQ_ERR_DEVICE, QLQ_ERR_HIP,
    QLQ_F32, QLQ_F16, QLQ_BF16, DTYPE_CODE, SIGNATURES,
    lib, lib_path, last_error,
    qlq_pack, qlq_unpack, qlq_dequantize, qlq_linear_workspace_size, qlq_linear_forward,
    qlq_set_skinny_max_m, qlq_get_skinny_max_m,
    bitlinear_pack, bitlinear_forward,
    qlq_quantize_rows_int8, qlq_quantize_rows_int8_clip, qlq_int8_matmul_int32, w8a8_workspace_size, w8a8_linear_forward,
    w8a8_linear_forward_noalloc, W8A8_NOALLOC_SCRATCH_BYTES,
    qlq_set_w8a8_fused_quant, qlq_get_w8a8_fused_quant,
    qlq_quantize_groups_int8, pergroup_workspace_size, pergroup_linear_forward,
    w4a8_pack_weight_int4, w4a8_workspace_size, w4a8_linear_forward,
    qlq_device_check, qlq_version,
)
