"""mamba2_scan_bwd_full: the backward and the input gradients together, on an MI355X.

Every output must agree with mamba2_scan_bwd (dW_A, dW_B, dW_C) followed by
mamba2_scan_bwd_input (d_h_history, d_h_s2) to fp32 rounding, hold the
accuracy of fp32 arithmetic against the oracle, and be bitwise reproducible.
At STATE_D = 16 both come from one pass: the backward's work-groups multiply
each unit's d_a, d_b, d_c into the weights of their column block, on bf16
MFMAs against exact three-term splits of both operands, and with fp32 trunk
inputs they sum their split-K partials over 8 waves instead of 12 (another
fixed order).  At other widths the two kernels run in sequence.  Parity with the oracle uses the path's tolerances
(outputs elementwise 1e-4 (1 + |ref|), weight gradients 1e-3 L1-relative).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_mamba2_scan_amd as m2
from oracle import mamba2_oracle as orc
from tests.inputs import bf16_round, make_inputs, workload_inputs
from tests.shapes import EDGE_SHAPES, LONG_FEW_SHAPES, gate_bias
from tests.test_parity_gpu import _to_dev, assert_elementwise, assert_l1

pytestmark = pytest.mark.gpu


def _separate(t, saved, K):
    g = m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"])
    dH, dhs2 = m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, t["d_context"], K)
    return {**g, "d_h_history": dH, "d_h_s2": dhs2}


def _full(t, saved, **kw):
    return m2.bwd_full(t["h_history"], t["h_s2"], saved, t["d_context"], t["W_A"], t["W_B"], t["W_C"], **kw)


def _same_bits(a, b, where):
    """Every output to fp32 rounding of the two separate calls."""
    for k in ("d_h_history", "d_h_s2"):
        assert_elementwise(a[k].cpu().numpy(), b[k].cpu().numpy().astype(np.float64), f"{k} {where}", tol=1e-5)
    for k in ("dW_A", "dW_B", "dW_C"):
        assert_l1(a[k].cpu().numpy(), b[k].cpu().numpy().astype(np.float64), f"{k} {where}", tol=1e-5)


def _oracle_check(got, inputs):
    _, b = orc.fwd_bwd(inputs)
    for k in ("dW_A", "dW_B", "dW_C"):
        assert_l1(got[k].cpu().numpy(), getattr(b, k), k)
    ig = orc.input_grads(b, inputs["W_A"], inputs["W_B"], inputs["W_C"])
    assert_elementwise(got["d_h_history"].cpu().numpy(), ig.d_h_history, "d_h_history")
    assert_elementwise(got["d_h_s2"].cpu().numpy(), ig.d_h_s2, "d_h_s2")


@pytest.mark.parametrize("B,K,SH2,D", EDGE_SHAPES + [(2050, 3, 320, 16), (1000, 48, 256, 16)], ids=lambda v: str(v))
def test_full_equals_separate_calls_and_oracle(B, K, SH2, D):
    inputs = make_inputs(B, K, SH2, D, seed=B + 5 * K + 3, gate_bias=gate_bias(K))
    t = _to_dev(inputs)
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    full = _full(t, saved)
    sep = _separate(t, saved, K)
    torch.cuda.synchronize()
    _same_bits(full, sep, (B, K, SH2, D))
    _oracle_check(full, inputs)


@pytest.mark.parametrize("B,K,SH2,D", LONG_FEW_SHAPES[:4], ids=lambda v: str(v))
def test_full_chunked_history(B, K, SH2, D):
    """Few samples, long histories: unit slices that start and end inside a block."""
    inputs = make_inputs(B, K, SH2, D, seed=B + K + 13, gate_bias=2.0)
    t = _to_dev(inputs)
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    full = _full(t, saved)
    sep = _separate(t, saved, K)
    torch.cuda.synchronize()
    _same_bits(full, sep, (B, K, SH2, D))
    _oracle_check(full, inputs)


@pytest.mark.parametrize("B,K,SH2,D", [(33, 9, 256, 16), (300, 12, 192, 16), (40, 8, 320, 64)],
                         ids=lambda v: str(v))
def test_full_bf16_trunk(B, K, SH2, D):
    """bf16 h_history / h_s2, against the two separate bf16 calls."""
    inputs = make_inputs(B, K, SH2, D, seed=B + K + 29)
    dev = torch.device("cuda:0")
    t = _to_dev(inputs)
    host = dict(inputs)
    for k in ("h_history", "h_s2"):
        bits, host[k] = bf16_round(inputs[k])
        t[k] = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    full = _full(t, saved)
    sep = _separate(t, saved, K)
    torch.cuda.synchronize()
    _same_bits(full, sep, (B, K, SH2, D))
    _oracle_check(full, host)


def test_full_workload_pages_shape():
    """The pages' shape at full size, against the two calls; the oracle on
    every weight gradient and on 512 sampled rows of each input gradient."""
    inputs = workload_inputs("pages_shape")
    t = _to_dev(inputs)
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    full = _full(t, saved)
    sep = _separate(t, saved, 8)
    torch.cuda.synchronize()
    _same_bits(full, sep, "pages_shape")
    _, b = orc.fwd_bwd(inputs)
    for k in ("dW_A", "dW_B", "dW_C"):
        assert_l1(full[k].cpu().numpy(), getattr(b, k), k)
    rng = np.random.default_rng(3)
    B = inputs["h_history"].shape[0]
    rows = np.unique(np.concatenate([np.arange(16), np.arange(B - 16, B), rng.choice(B, 480, replace=False)]))
    import dataclasses
    bs = dataclasses.replace(b, d_a=b.d_a[rows], d_b=b.d_b[rows], d_c=b.d_c[rows])
    ig = orc.input_grads(bs, inputs["W_A"], inputs["W_B"], inputs["W_C"])
    idx = torch.from_numpy(rows).to(saved.device)
    assert_elementwise(full["d_h_history"].index_select(0, idx).cpu().numpy(), ig.d_h_history, "d_h_history")
    assert_elementwise(full["d_h_s2"].index_select(0, idx).cpu().numpy(), ig.d_h_s2, "d_h_s2")


def test_full_bitwise_reproducible():
    inputs = make_inputs(1000, 9, 256, 16, seed=8)
    t = _to_dev(inputs)
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    a = _full(t, saved)
    b = _full(t, saved)
    torch.cuda.synchronize()
    for k in ("dW_A", "dW_B", "dW_C", "d_h_history", "d_h_s2"):
        assert torch.equal(a[k], b[k]), k


def test_full_one_output_and_overwrite():
    """Either input gradient alone; pre-filled outputs are overwritten."""
    inputs = make_inputs(77, 9, 192, 16, seed=5)
    t = _to_dev(inputs)
    dev = t["W_A"].device
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    sep = _separate(t, saved, 9)
    only_h = _full(t, saved, out={"d_h_history": torch.full((77, 9, 192), float("nan"), device=dev)},
                   want=("h_history",))
    only_s = _full(t, saved, out={"d_h_s2": torch.full((77, 192), float("nan"), device=dev)}, want=("h_s2",))
    torch.cuda.synchronize()
    assert only_h["d_h_s2"] is None and only_s["d_h_history"] is None
    full = _full(t, saved)
    torch.cuda.synchronize()
    assert torch.equal(only_h["d_h_history"], full["d_h_history"])
    assert torch.equal(only_s["d_h_s2"], full["d_h_s2"])
    assert_elementwise(only_h["d_h_history"].cpu().numpy(), sep["d_h_history"].cpu().numpy().astype(np.float64),
                       "d_h_history", tol=1e-5)
    for k in ("dW_A", "dW_B", "dW_C"):
        assert torch.equal(only_h[k], only_s[k]), k
        assert_l1(only_h[k].cpu().numpy(), sep[k].cpu().numpy().astype(np.float64), k, tol=1e-5)


@pytest.mark.parametrize("shape", [(300, 8, 256, 16), (300, 64, 256, 16), (40, 20, 192, 16)],
                         ids=["K8", "K64", "rounds"])
def test_full_fp32_class_accuracy(shape):
    """The one-pass input gradients hold fp32 accuracy: elementwise error /
    (1 + |ref|) <= 5e-6 against the fp64 oracle (two-term splits, 2^-17 per
    product, would give ~1e-5)."""
    B, K, SH2, D = shape
    inputs = make_inputs(B, K, SH2, D, seed=17)
    t = _to_dev(inputs)
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    full = _full(t, saved)
    torch.cuda.synchronize()
    _, b = orc.fwd_bwd(inputs)
    ig = orc.input_grads(b, inputs["W_A"], inputs["W_B"], inputs["W_C"])
    for name, ref in (("d_h_history", ig.d_h_history), ("d_h_s2", ig.d_h_s2)):
        got = full[name].cpu().numpy().astype(np.float64)
        worst = float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))
        assert worst <= 5e-6, f"{name}: {worst:.3e}"
    for k in ("dW_A", "dW_B", "dW_C"):
        ref = getattr(b, k)
        rel = float(np.sum(np.abs(full[k].cpu().numpy().astype(np.float64) - ref)) / np.sum(np.abs(ref)))
        assert rel <= 3e-6, f"{k}: {rel:.3e}"
