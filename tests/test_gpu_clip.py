"""GPU parity for the percentile-clipped per-row int8 quantizer
(qlq_quantize_rows_int8_clip): bit-exact codes and scales against the
oracle, including ties at the percentile index, zero clips, zero rows, p = 0
and 100, rows shorter and longer than a power of two, and every input dtype."""

import numpy as np
import pytest
import torch

import oracle
import bit_weight_quantized_qlq_amd as qlq
from parity import dev, f32

pytestmark = pytest.mark.gpu


def _check(w_t, p):
    q, s = qlq.qlq_quantize_rows_int8_clip(w_t.to(dev()), p)
    q_ref, s_ref = oracle.quantize_rows_int8_clip(f32(w_t), p)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), p
    assert np.array_equal(q.cpu().numpy(), q_ref), p


@pytest.mark.parametrize("vdt", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("K", [1, 5, 100, 1000, 4096, 16384])
def test_random_rows(vdt, K):
    rng = np.random.default_rng(K)
    w = (rng.standard_normal((13, K)) * rng.uniform(1e-2, 10, size=(13, 1))).astype(np.float32)
    w[2] = 0                                             # zero row: scale 1
    w[3, : max(1, K * 3 // 4)] = 0                       # percentile lands on zeros: absmax fallback
    w[4, ::3] *= 40                                      # outliers
    w[5] = np.round(w[5])                                # many equal magnitudes
    wt = torch.from_numpy(w).to(vdt)
    for p in (0.0, 25.0, 50.0, 87.5, 99.0, 99.9, 100.0):
        _check(wt, p)


def test_workload_weights():
    import workloads
    w = workloads.w8a8_inputs(1, 4096, 4096, seed=1005)["w"]
    for p in (99.9, 99.99):
        _check(w, p)


def test_clipped_weights_run_through_w8a8():
    """The clip quantizer's output is an ordinary W8A8 weight."""
    import workloads
    from parity import assert_close
    inp = workloads.w8a8_inputs(64, 1024, 256, seed=9)
    wq, sw = qlq.qlq_quantize_rows_int8_clip(inp["w"].to(dev()), 99.9)
    wq_ref, sw_ref = oracle.quantize_rows_int8_clip(inp["w"].numpy(), 99.9)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), sw_ref.view(np.uint32))
    y = qlq.w8a8_linear_forward(inp["x"].to(dev()), wq, sw)
    _, _, _, y_ref, D = oracle.w8a8_forward(f32(inp["x"]), wq_ref, sw_ref)
    assert_close(y, y_ref, D, 1024, torch.float16, label="w8a8 on clipped weights")
