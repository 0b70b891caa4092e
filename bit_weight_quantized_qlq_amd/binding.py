"""ctypes binding of libqlq (include/qlq.h), one Python function per entry point.

The binding only marshals arguments: it checks that tensors live on a HIP
device with the dtype and layout the C ABI expects, allocates outputs with
torch (when the caller passes none), passes raw device pointers and the
current torch stream, and turns a non-zero status into ``QLQError``.  Every
step of the computation runs in the library's HIP kernels.  If the library is
not built, importing works but the first call raises.
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlq.so")

QLQ_OK = 0
QLQ_ERR_INVALID_ARG = 1
QLQ_ERR_UNSUPPORTED = 2
QLQ_ERR_DTYPE = 3
QLQ_ERR_ALIGNMENT = 4
QLQ_ERR_WORKSPACE = 5
QLQ_ERR_DATA = 6
QLQ_ERR_DEVICE = 7
QLQ_ERR_HIP = 8

QLQ_F32, QLQ_F16, QLQ_BF16 = 0, 1, 2
DTYPE_CODE = {torch.float32: QLQ_F32, torch.float16: QLQ_F16, torch.bfloat16: QLQ_BF16}


class QLQError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"qlq error {code}: {message}")
        self.code = code


_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/qlq.h
SIGNATURES = {
    "qlq_pack": (_int, [_vp, _i64, _i64, _int, _int, _vp, _vp, _vp, _int, _vp]),
    "qlq_unpack": (_int, [_vp, _i64, _i64, _int, _vp, _vp]),
    "qlq_dequantize": (_int, [_vp, _vp, _vp, _int, _i64, _i64, _int, _int, _vp, _vp]),
    "qlq_linear_workspace_size": (_sz, [_i64, _i64, _i64, _int, _int, _int]),
    "qlq_linear_forward": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _int, _i64, _int, _int, _vp,
                                  _vp, _vp, _sz, _vp]),
    "qlq_set_skinny_max_m": (_int, [_int]),
    "qlq_get_skinny_max_m": (_int, []),
    "qlq_set_w8a8_fused_quant": (_int, [_int]),
    "qlq_get_w8a8_fused_quant": (_int, []),
    "bitlinear_pack": (_int, [_vp, _i64, _i64, _vp, _vp]),
    "bitlinear_forward": (_int, [_vp, _int, _i64, _i64, _vp, _i64, _vp, _int, _vp, _vp, _vp]),
    "qlq_quantize_rows_int8": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp]),
    "qlq_quantize_rows_int8_clip": (_int, [_vp, _int, _i64, _i64, ctypes.c_float, _vp, _vp, _vp]),
    "qlq_int8_matmul_int32": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "w8a8_workspace_size": (_sz, [_i64, _i64]),
    "w8a8_linear_forward": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "w8a8_linear_forward_noalloc": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp]),
    "qlq_quantize_groups_int8": (_int, [_vp, _int, _i64, _i64, _int, _vp, _vp, _vp]),
    "pergroup_workspace_size": (_sz, [_i64, _i64]),
    "pergroup_linear_forward": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _i64, _int, _vp, _vp, _vp, _sz, _vp]),
    "w4a8_pack_weight_int4": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp]),
    "w4a8_workspace_size": (_sz, [_i64, _i64, _i64]),
    "w4a8_linear_forward": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "qlq_device_check": (_int, [_int]),
    "qlq_last_error": (ctypes.c_char_p, []),
    "qlq_version": (ctypes.c_char_p, []),
}

_lib = None


def lib_path():
    return _LIB_PATH


def lib():
    """The loaded libqlq.so (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m bit_weight_quantized_qlq_amd.build`")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error():
    return lib().qlq_last_error().decode()


def _check(status):
    if status != QLQ_OK:
        raise QLQError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise QLQError(QLQ_ERR_DTYPE, f"{name} has dtype {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    return t


def _flatten(x):
    return x.reshape(-1, x.shape[-1]) if x.dim() != 2 else x


def _shape(t, name, shape):
    """Raise ValueError unless tensor ``t`` has exactly ``shape``."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _out_shape(out, M, N):
    """An output tensor must hold exactly M*N elements with N innermost."""
    if out is not None and (out.numel() != M * N or (out.dim() and out.shape[-1] != N)):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {M * N} elements as [..., {N}]")


def _whole_groups(K, group_size):
    return group_size > 0 and K % group_size == 0


def _check_affine_operands(K, packed, scales, biases, bits, group_size):
    """packed [N, K*bits/32]; scales and biases [N, K/group_size].  Shapes the
    library rejects anyway (K not a whole number of words or groups) are left
    to its own error codes."""
    if packed.dim() != 2:
        raise ValueError("packed must be 2-D")
    N = packed.shape[0]
    if bits > 0 and (K * bits) % 32 == 0:
        _shape(packed, "packed", (N, K * bits // 32))
    if _whole_groups(K, group_size):
        _shape(scales, "scales", (N, K // group_size))
        _shape(biases, "biases", (N, K // group_size))
    return N


# ------------------------------------------------------------------ affine
def qlq_pack(w, bits=4, group_size=64, sb_dtype=torch.bfloat16):
    """Quantize fp32 weights [N, K]; returns (packed uint32 as int32, scales, biases)."""
    _dev(w, "w", torch.float32, 2)
    N, K = w.shape
    packed = torch.empty((N, K * bits // 32), dtype=torch.int32, device=w.device)
    scales = torch.empty((N, K // group_size), dtype=sb_dtype, device=w.device)
    biases = torch.empty_like(scales)
    _check(lib().qlq_pack(_ptr(w), N, K, bits, group_size, _ptr(packed), _ptr(scales), _ptr(biases),
                          DTYPE_CODE[sb_dtype], _stream(w)))
    return packed, scales, biases


def qlq_unpack(packed, K, bits=4):
    if packed.dim() == 2 and bits > 0 and (K * bits) % 32 == 0:
        _shape(packed, "packed", (packed.shape[0], K * bits // 32))
    _dev(packed, "packed", torch.int32, 2)
    N = packed.shape[0]
    codes = torch.empty((N, K), dtype=torch.uint8, device=packed.device)
    _check(lib().qlq_unpack(_ptr(packed), N, K, bits, _ptr(codes), _stream(packed)))
    return codes


def qlq_dequantize(packed, scales, biases, K, bits=4, group_size=64):
    _check_affine_operands(K, packed, scales, biases, bits, group_size)
    _dev(packed, "packed", torch.int32, 2)
    _dev(scales, "scales", tuple(DTYPE_CODE))
    _dev(biases, "biases", scales.dtype)
    N = packed.shape[0]
    w = torch.empty((N, K), dtype=torch.float32, device=packed.device)
    _check(lib().qlq_dequantize(_ptr(packed), _ptr(scales), _ptr(biases), DTYPE_CODE[scales.dtype], N, K,
                                bits, group_size, _ptr(w), _stream(packed)))
    return w


def qlq_linear_workspace_size(M, K, N, bits, group_size, x_dtype):
    return int(lib().qlq_linear_workspace_size(M, K, N, bits, group_size, DTYPE_CODE[x_dtype]))


def qlq_linear_forward(x, packed, scales, biases, bits=4, group_size=64, bias=None, out=None,
                       workspace=None):
    """y = x . dequant(W)^T (+ bias) over the last axis of x."""
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    N = _check_affine_operands(K, packed, scales, biases, bits, group_size)
    _shape(bias, "bias", (N,))
    _out_shape(out, M, N)
    _dev(x, "x", tuple(DTYPE_CODE))
    _dev(packed, "packed", torch.int32, 2)
    _dev(scales, "scales")
    _dev(biases, "biases")
    if bias is not None:
        _dev(bias, "bias", x.dtype, 1)
    x2 = _flatten(x)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _dev(out, "out", x.dtype)
    need = qlq_linear_workspace_size(M, K, N, bits, group_size, x.dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qlq_linear_forward(_ptr(x2), DTYPE_CODE[x.dtype], M, K, _ptr(packed), _ptr(scales),
                                    _ptr(biases), DTYPE_CODE.get(scales.dtype, -1), N, bits, group_size,
                                    _ptr(bias), _ptr(out), _ptr(workspace), ws_bytes, _stream(x)))
    return out.reshape(*x.shape[:-1], N)


def qlq_set_skinny_max_m(m):
    _check(lib().qlq_set_skinny_max_m(m))


def qlq_get_skinny_max_m():
    return int(lib().qlq_get_skinny_max_m())


# ----------------------------------------------------------------- ternary
def bitlinear_pack(t):
    """Ternary int8 [N, K] in {-1, 0, 1} -> packed uint8 [N/4, K]."""
    _dev(t, "t", torch.int8, 2)
    N, K = t.shape
    packed = torch.empty((N // 4, K), dtype=torch.uint8, device=t.device)
    _check(lib().bitlinear_pack(_ptr(t), N, K, _ptr(packed), _stream(t)))
    return packed


def bitlinear_forward(x, packed, N, weight_scale, invert_weight_scale=False, bias=None, out=None):
    """y = sigma * x . decode(packed)^T (+ bias); weight_scale must have x's dtype."""
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if N % 4 == 0:
        _shape(packed, "packed", (N // 4, K))
    if weight_scale.numel() != 1:
        raise ValueError(f"weight_scale must hold one element, not {weight_scale.numel()}")
    _shape(bias, "bias", (N,))
    _out_shape(out, M, N)
    _dev(x, "x", tuple(DTYPE_CODE))
    _dev(packed, "packed", torch.uint8, 2)
    _dev(weight_scale, "weight_scale", x.dtype)
    if bias is not None:
        _dev(bias, "bias", x.dtype, 1)
    x2 = _flatten(x)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _dev(out, "out", x.dtype)
    _check(lib().bitlinear_forward(_ptr(x2), DTYPE_CODE[x.dtype], M, K, _ptr(packed), N, _ptr(weight_scale),
                                   int(bool(invert_weight_scale)), _ptr(bias), _ptr(out), _stream(x)))
    return out.reshape(*x.shape[:-1], N)


# -------------------------------------------------------------------- W8A8
def qlq_quantize_rows_int8(v):
    _dev(v, "v", tuple(DTYPE_CODE), 2)
    R, K = v.shape
    q = torch.empty((R, K), dtype=torch.int8, device=v.device)
    s = torch.empty((R,), dtype=torch.float32, device=v.device)
    _check(lib().qlq_quantize_rows_int8(_ptr(v), DTYPE_CODE[v.dtype], R, K, _ptr(q), _ptr(s), _stream(v)))
    return q, s


def qlq_quantize_rows_int8_clip(v, clip_percentile):
    """Per-row int8 with the clip at a percentile of |v|: v [R, K] -> (q int8, scale f32 [R])."""
    _dev(v, "v", tuple(DTYPE_CODE), 2)
    R, K = v.shape
    q = torch.empty((R, K), dtype=torch.int8, device=v.device)
    s = torch.empty((R,), dtype=torch.float32, device=v.device)
    _check(lib().qlq_quantize_rows_int8_clip(_ptr(v), DTYPE_CODE[v.dtype], R, K, float(clip_percentile), _ptr(q),
                                             _ptr(s), _stream(v)))
    return q, s


def qlq_int8_matmul_int32(a, b):
    _dev(a, "a", torch.int8, 2)
    _dev(b, "b", torch.int8, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    c = torch.empty((M, N), dtype=torch.int32, device=a.device)
    _check(lib().qlq_int8_matmul_int32(_ptr(a), _ptr(b), M, N, K, _ptr(c), _stream(a)))
    return c


def qlq_set_w8a8_fused_quant(on):
    """Select where the W8A8 activation quantizer runs: 0 before the GEMM
    (default), 1 inside it (bit-identical results)."""
    _check(lib().qlq_set_w8a8_fused_quant(int(on)))


def qlq_get_w8a8_fused_quant():
    return int(lib().qlq_get_w8a8_fused_quant())


def w8a8_workspace_size(M, K):
    return int(lib().w8a8_workspace_size(M, K))


def w8a8_linear_forward(x, w, scale_w, bias=None, out=None, workspace=None):
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if w.dim() != 2:
        raise ValueError("w must be 2-D")
    N = w.shape[0]
    _shape(w, "w", (N, K))
    _shape(scale_w, "scale_w", (N,))
    _shape(bias, "bias", (N,))
    _out_shape(out, M, N)
    _dev(x, "x", (torch.float16, torch.bfloat16))
    _dev(w, "w", torch.int8, 2)
    _dev(scale_w, "scale_w", torch.float32, 1)
    if bias is not None:
        _dev(bias, "bias", x.dtype, 1)
    x2 = _flatten(x)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _dev(out, "out", x.dtype)
    need = w8a8_workspace_size(M, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().w8a8_linear_forward(_ptr(x2), DTYPE_CODE[x.dtype], M, K, _ptr(w), _ptr(scale_w), N,
                                     _ptr(bias), _ptr(out), _ptr(workspace), ws_bytes, _stream(x)))
    return out.reshape(*x.shape[:-1], N)


# Scratch bytes the allocation-free W8A8 call holds on each GPU
# (QLQ_W8A8_NOALLOC_SCRATCH_BYTES in include/qlq.h).
W8A8_NOALLOC_SCRATCH_BYTES = 16 << 20


def w8a8_linear_forward_noalloc(x, w, scale_w, bias=None, out=None):
    """w8a8_linear_forward without a workspace: the library's static device
    scratch holds the quantized activations.  The binding allocates ``out``
    when none is given; pass ``out`` to keep the call free of allocations.
    Calls that overlap on one GPU race on the shared scratch."""
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if w.dim() != 2:
        raise ValueError("w must be 2-D")
    N = w.shape[0]
    _shape(w, "w", (N, K))
    _shape(scale_w, "scale_w", (N,))
    _shape(bias, "bias", (N,))
    _out_shape(out, M, N)
    _dev(x, "x", (torch.float16, torch.bfloat16))
    _dev(w, "w", torch.int8, 2)
    _dev(scale_w, "scale_w", torch.float32, 1)
    if bias is not None:
        _dev(bias, "bias", x.dtype, 1)
    x2 = _flatten(x)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _dev(out, "out", x.dtype)
    _check(lib().w8a8_linear_forward_noalloc(_ptr(x2), DTYPE_CODE[x.dtype], M, K, _ptr(w), _ptr(scale_w), N,
                                             _ptr(bias), _ptr(out), _stream(x)))
    return out.reshape(*x.shape[:-1], N)


# --------------------------------------------------------- per-group int8
def qlq_quantize_groups_int8(w, group_size):
    """Per-group symmetric int8: w [N, K] -> (q int8 [N, K], scale f32 [K/group_size, N])."""
    _dev(w, "w", tuple(DTYPE_CODE), 2)
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.int8, device=w.device)
    s = torch.empty((K // group_size if group_size > 0 else 0, N), dtype=torch.float32, device=w.device)
    _check(lib().qlq_quantize_groups_int8(_ptr(w), DTYPE_CODE[w.dtype], N, K, group_size, _ptr(q), _ptr(s),
                                          _stream(w)))
    return q, s


def pergroup_workspace_size(M, K):
    return int(lib().pergroup_workspace_size(M, K))


def pergroup_linear_forward(x, w, scale_w, group_size, bias=None, out=None, workspace=None):
    """Per-group int8 linear; M == 1 keeps x in floating point, M > 1 quantizes it."""
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if w.dim() != 2:
        raise ValueError("w must be 2-D")
    N = w.shape[0]
    _shape(w, "w", (N, K))
    if _whole_groups(K, group_size):
        _shape(scale_w, "scale_w", (K // group_size, N))
    _shape(bias, "bias", (N,))
    _out_shape(out, M, N)
    _dev(x, "x", (torch.float16, torch.bfloat16))
    _dev(w, "w", torch.int8, 2)
    _dev(scale_w, "scale_w", torch.float32, 2)
    if bias is not None:
        _dev(bias, "bias", x.dtype, 1)
    x2 = _flatten(x)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _dev(out, "out", x.dtype)
    need = pergroup_workspace_size(M, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pergroup_linear_forward(_ptr(x2), DTYPE_CODE[x.dtype], M, K, _ptr(w), _ptr(scale_w), N,
                                         group_size, _ptr(bias), _ptr(out), _ptr(workspace), ws_bytes,
                                         _stream(x)))
    return out.reshape(*x.shape[:-1], N)


# ------------------------------------------------ per-column int4, W4A8
def w4a8_pack_weight_int4(w):
    """Per-column symmetric int4: w [K, N] -> (packed uint8 [K/2, N], scale f32 [N])."""
    _dev(w, "w", tuple(DTYPE_CODE), 2)
    K, N = w.shape
    packed = torch.empty((K // 2, N), dtype=torch.uint8, device=w.device)
    s = torch.empty((N,), dtype=torch.float32, device=w.device)
    _check(lib().w4a8_pack_weight_int4(_ptr(w), DTYPE_CODE[w.dtype], K, N, _ptr(packed), _ptr(s), _stream(w)))
    return packed, s


def w4a8_workspace_size(M, K, N):
    return int(lib().w4a8_workspace_size(M, K, N))


def w4a8_linear_forward(x, packed_w, scale_w, bias=None, out=None, workspace=None):
    """W4A8 linear: x [..., K] f16/bf16, packed_w uint8 [K/2, N], scale_w f32 [N]."""
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    if packed_w.dim() != 2:
        raise ValueError("packed_w must be 2-D")
    N = packed_w.shape[1]
    if packed_w.shape[0] * 2 != K:
        raise ValueError("packed_w must be [K/2, N]")
    _shape(scale_w, "scale_w", (N,))
    _shape(bias, "bias", (N,))
    _out_shape(out, M, N)
    _dev(x, "x", (torch.float16, torch.bfloat16))
    _dev(packed_w, "packed_w", torch.uint8, 2)
    _dev(scale_w, "scale_w", torch.float32, 1)
    if bias is not None:
        _dev(bias, "bias", x.dtype, 1)
    x2 = _flatten(x)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _dev(out, "out", x.dtype)
    need = w4a8_workspace_size(M, K, N)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().w4a8_linear_forward(_ptr(x2), DTYPE_CODE[x.dtype], M, K, _ptr(packed_w), _ptr(scale_w), N,
                                     _ptr(bias), _ptr(out), _ptr(workspace), ws_bytes, _stream(x)))
    return out.reshape(*x.shape[:-1], N)


# ------------------------------------------------------------------ device
def qlq_device_check(device=0):
    return int(lib().qlq_device_check(device))


def qlq_version():
    return lib().qlq_version().decode()
