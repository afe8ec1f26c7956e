"""The bfloat16 trunk-input entry points (h_history, h_s2 as bf16) on an MI355X.

The oracle runs on the same bf16-rounded values, so the tolerances are the
fp32 path's.  Both passes multiply the bf16 values with bf16 MFMAs against
the other operand split exactly into three bf16 terms (the weights in the
forward, d_a/d_b/d_c in the backward): every product is exact and the sums
run in fp32, in another order than the fp32 path's, so against the fp32
entry points fed the widened values the results agree to fp32 rounding
(checked at 1e-5).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_mamba2_scan_amd as m2
from oracle import mamba2_oracle as orc
from tests.inputs import bf16_round, make_inputs, workload_inputs
from tests.shapes import BF16_CHUNKED_SHAPES, BF16_WORKLOADS, EDGE_SHAPES, FORM_SHAPES, gate_bias
from tests.test_parity_gpu import assert_elementwise, assert_l1

pytestmark = pytest.mark.gpu


def split(inputs):
    """(bf16 device tensors, fp32 device tensors of the same values, host inputs with those values)."""
    dev = torch.device("cuda:0")
    host = dict(inputs)
    t16, t32 = {}, {}
    for k in ("h_history", "h_s2"):
        bits, vals = bf16_round(inputs[k])
        host[k] = vals
        t16[k] = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        t32[k] = torch.from_numpy(vals).to(dev)
    for k in ("W_A", "W_B", "W_C", "d_context"):
        t16[k] = t32[k] = torch.from_numpy(inputs[k]).to(dev)
    return t16, t32, host


def run(t, debug):
    ctx, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    g = m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"], debug=debug)
    torch.cuda.synchronize()
    return ctx, saved, g


def check(inputs, debug=True):
    t16, t32, host = split(inputs)
    assert t16["h_history"].dtype == torch.bfloat16
    ctx, saved, g = run(t16, debug)
    f, b = orc.fwd_bwd(host)
    assert_elementwise(ctx.cpu().numpy(), f.context, "context")
    for name in ("dW_A", "dW_B", "dW_C"):
        assert_l1(g[name].cpu().numpy(), getattr(b, name), name)
    if debug:
        for name in ("d_a", "d_b", "d_c"):
            assert_elementwise(g[name].cpu().numpy(), getattr(b, name), name)
    # the same values through the fp32 entry points
    ctx32, saved32, g32 = run(t32, debug)
    assert_elementwise(ctx.cpu().numpy(), ctx32.cpu().numpy().astype(np.float64), "context vs fp32 path", tol=1e-5)
    for name in ("dW_A", "dW_B", "dW_C"):
        assert_l1(g[name].cpu().numpy(), g32[name].cpu().numpy().astype(np.float64), name + " vs fp32 path", tol=1e-5)
    # the backward alone, on one forward's saved terms: fp32 rounding apart
    g16b = m2.bwd(t16["h_history"], t16["h_s2"], saved32, t16["d_context"])
    g32b = m2.bwd(t32["h_history"], t32["h_s2"], saved32, t32["d_context"])
    torch.cuda.synchronize()
    for name in ("dW_A", "dW_B", "dW_C"):
        assert_l1(g16b[name].cpu().numpy(), g32b[name].cpu().numpy().astype(np.float64), name + " (bwd alone)",
                  tol=1e-5)


@pytest.mark.parametrize("B,K,SH2,D", EDGE_SHAPES, ids=lambda v: str(v))
def test_bf16_edge_shapes(B, K, SH2, D):
    check(make_inputs(B, K, SH2, D, seed=B * 3 + K + 2))


@pytest.mark.parametrize("name", BF16_WORKLOADS[:3])
def test_bf16_workloads(name):
    check(workload_inputs(name), debug=(name != "pages_shape"))


@pytest.mark.parametrize("name", BF16_WORKLOADS[3:])
def test_bf16_large(name):
    check(workload_inputs(name), debug=False)


@pytest.mark.parametrize("B,K,SH2,D", BF16_CHUNKED_SHAPES, ids=lambda v: str(v))
def test_bf16_chunked_history(B, K, SH2, D):
    """Few samples, long histories: the chunked forward (summary, carry, replay) with bf16 inputs."""
    check(make_inputs(B, K, SH2, D, seed=B + K + 5, gate_bias=2.0), debug=(K <= 300))


@pytest.mark.parametrize("B,K,SH2,D", FORM_SHAPES, ids=lambda v: str(v))
def test_bf16_launch_forms(B, K, SH2, D):
    """The wide-trunk launch forms (two-block full and summary passes, one-block
    summary passes, two-block replays) with bf16 inputs."""
    check(make_inputs(B, K, SH2, D, seed=B + 3 * K + SH2 + 1, gate_bias=gate_bias(K)))


def test_bf16_split_phase_matches():
    inputs = make_inputs(300, 9, 192, 32, seed=77)
    t16, _, _ = split(inputs)
    ctx, saved = m2.fwd(t16["h_history"], t16["h_s2"], t16["W_A"], t16["W_B"], t16["W_C"])
    full = m2.bwd(t16["h_history"], t16["h_s2"], saved, t16["d_context"])
    ws = m2.alloc_workspace(300, 9, 192, 32, ctx.device)
    m2.bwd_partials(t16["h_history"], t16["h_s2"], saved, t16["d_context"], ws)
    parts = {n: torch.empty_like(full[n]) for n in ("dW_A", "dW_B", "dW_C")}
    m2.bwd_reduce(300, 9, 192, 32, ws, parts["dW_A"], parts["dW_B"], parts["dW_C"])
    torch.cuda.synchronize()
    for n in parts:
        assert torch.equal(parts[n], full[n]), n


def test_bf16_mixed_dtypes_rejected():
    inputs = make_inputs(20, 4, 128, 16, seed=5)
    t16, t32, _ = split(inputs)
    with pytest.raises(TypeError):
        m2.fwd(t16["h_history"], t32["h_s2"], t16["W_A"], t16["W_B"], t16["W_C"])
