"""The Python binding's argument checks, on the CPU: every forward binding
compares each tensor's shape with the (M, K, N, bits, group_size) it passes to
the C ABI and raises ValueError before any library call when they disagree.

The library handle is replaced by a recorder, so a test also shows that no C
entry point was reached.  Tensors live on the CPU: the shape checks run before
the device checks, and a well-shaped call gets as far as the device check."""

import pytest
import torch

from bit_weight_quantized_qlq_amd import binding as B


class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture()
def rec(monkeypatch):
    r = _Recorder()
    monkeypatch.setattr(B, "_lib", r)
    return r


def _affine(M=3, K=256, N=40, bits=4, G=64, dt=torch.bfloat16):
    return dict(x=torch.zeros(M, K, dtype=dt), packed=torch.zeros(N, K * bits // 32, dtype=torch.int32),
                scales=torch.zeros(N, K // G, dtype=dt), biases=torch.zeros(N, K // G, dtype=dt))


def _raises_shape(rec, fn, *args, **kw):
    with pytest.raises(ValueError, match="shape|must be|expected|hold one"):
        fn(*args, **kw)
    assert rec.calls == [], rec.calls


def test_affine_forward_rejects_mismatched_shapes(rec):
    a = _affine()
    # scales packed with groups of 128 (the prefill layout), called with 64
    a128 = _affine(G=128)
    _raises_shape(rec, B.qlq_linear_forward, a["x"], a["packed"], a128["scales"], a["biases"], 4, 64)
    _raises_shape(rec, B.qlq_linear_forward, a["x"], a["packed"], a["scales"], a128["biases"], 4, 64)
    # packed for 3-bit codes, called with bits=4
    p3 = torch.zeros(40, 256 * 3 // 32, dtype=torch.int32)
    _raises_shape(rec, B.qlq_linear_forward, a["x"], p3, a["scales"], a["biases"], 4, 64)
    # packed from a K=512 weight with x of K=256
    _raises_shape(rec, B.qlq_linear_forward, a["x"], torch.zeros(40, 64, dtype=torch.int32),
                  a["scales"], a["biases"], 4, 64)
    _raises_shape(rec, B.qlq_linear_forward, a["x"], a["packed"], a["scales"], a["biases"], 4, 64,
                  bias=torch.zeros(39, dtype=torch.bfloat16))
    _raises_shape(rec, B.qlq_linear_forward, a["x"], a["packed"], a["scales"], a["biases"], 4, 64,
                  out=torch.zeros(3, 39, dtype=torch.bfloat16))
    _raises_shape(rec, B.qlq_linear_forward, a["x"], a["packed"], a["scales"], a["biases"], 4, 64,
                  out=torch.zeros(2, 40, dtype=torch.bfloat16))


def test_affine_helpers_reject_mismatched_shapes(rec):
    a = _affine()
    _raises_shape(rec, B.qlq_unpack, a["packed"], 512, 4)
    _raises_shape(rec, B.qlq_dequantize, a["packed"], a["scales"][:, :2], a["biases"], 256, 4, 64)


def test_well_shaped_affine_call_reaches_the_device_check(rec):
    a = _affine()
    with pytest.raises(ValueError, match="HIP device"):
        B.qlq_linear_forward(a["x"], a["packed"], a["scales"], a["biases"], 4, 64,
                             bias=torch.zeros(40, dtype=torch.bfloat16), out=torch.zeros(3, 40, dtype=torch.bfloat16))
    assert rec.calls == []


def test_bitlinear_rejects_mismatched_shapes(rec):
    x = torch.zeros(8, 128, dtype=torch.bfloat16)
    ws = torch.ones(1, dtype=torch.bfloat16)
    _raises_shape(rec, B.bitlinear_forward, x, torch.zeros(16, 128, dtype=torch.uint8), 68, ws)   # N/4 = 17
    _raises_shape(rec, B.bitlinear_forward, x, torch.zeros(17, 96, dtype=torch.uint8), 68, ws)    # K
    _raises_shape(rec, B.bitlinear_forward, x, torch.zeros(17, 128, dtype=torch.uint8), 68,
                  torch.ones(2, dtype=torch.bfloat16))
    _raises_shape(rec, B.bitlinear_forward, x, torch.zeros(17, 128, dtype=torch.uint8), 68, ws,
                  bias=torch.zeros(64, dtype=torch.bfloat16))
    _raises_shape(rec, B.bitlinear_forward, x, torch.zeros(17, 128, dtype=torch.uint8), 68, ws,
                  out=torch.zeros(8, 64, dtype=torch.bfloat16))


def test_w8a8_rejects_mismatched_shapes(rec):
    x = torch.zeros(4, 256, dtype=torch.float16)
    w = torch.zeros(48, 256, dtype=torch.int8)
    sw = torch.ones(48)
    _raises_shape(rec, B.w8a8_linear_forward, x, torch.zeros(48, 128, dtype=torch.int8), sw)
    _raises_shape(rec, B.w8a8_linear_forward, x, w, torch.ones(47))
    _raises_shape(rec, B.w8a8_linear_forward, x, w, sw, bias=torch.zeros(47, dtype=torch.float16))
    _raises_shape(rec, B.w8a8_linear_forward, x, w, sw, out=torch.zeros(4, 47, dtype=torch.float16))


def test_pergroup_rejects_mismatched_shapes(rec):
    x = torch.zeros(4, 256, dtype=torch.float16)
    w = torch.zeros(48, 256, dtype=torch.int8)
    _raises_shape(rec, B.pergroup_linear_forward, x, w, torch.ones(4, 48), 128)     # scales of G = 64
    _raises_shape(rec, B.pergroup_linear_forward, x, w, torch.ones(48, 2), 128)     # untransposed
    _raises_shape(rec, B.pergroup_linear_forward, x, torch.zeros(48, 512, dtype=torch.int8), torch.ones(2, 48), 128)
    _raises_shape(rec, B.pergroup_linear_forward, x, w, torch.ones(2, 48), 128, bias=torch.zeros(4))


def test_w4a8_rejects_mismatched_shapes(rec):
    x = torch.zeros(4, 256, dtype=torch.float16)
    p = torch.zeros(128, 48, dtype=torch.uint8)
    _raises_shape(rec, B.w4a8_linear_forward, x, torch.zeros(64, 48, dtype=torch.uint8), torch.ones(48))
    _raises_shape(rec, B.w4a8_linear_forward, x, p, torch.ones(47))
    _raises_shape(rec, B.w4a8_linear_forward, x, p, torch.ones(48), bias=torch.zeros(47, dtype=torch.float16))
    _raises_shape(rec, B.w4a8_linear_forward, x, p, torch.ones(48), out=torch.zeros(5, 48, dtype=torch.float16))
