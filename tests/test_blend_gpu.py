"""Parity of the stability multiplier and the h_enriched blend against the CPU oracle.

mamba2_scan_fwd_blend (context, h_enriched) and mamba2_scan_bwd_blend
(d_context, dW_A, dW_B, dW_C, d_temporal_weight) through the C-ABI.
Tolerances as for the scan: outputs (context, h_enriched, d_context)
elementwise |gpu - ref| <= 1e-4 (1 + |ref|); gradients of weights (dW_*,
d_temporal_weight) sum|gpu - ref| / sum|ref| <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_mamba2_scan_amd as m2
from oracle import mamba2_oracle as orc
from tests.inputs import blend_extras, make_inputs, workload_inputs
from tests.shapes import EDGE_SHAPES
from tests.test_parity_gpu import _to_dev, assert_elementwise, assert_l1

pytestmark = pytest.mark.gpu


def run_blend(inputs, extras, m, with_w, rows=None):
    dev = torch.device("cuda:0")
    t = _to_dev(inputs)
    B, K, SH2 = inputs["h_history"].shape
    D = inputs["W_A"].shape[1]
    dhe = torch.from_numpy(extras["d_h_enriched"]).to(dev)
    w = torch.from_numpy(extras["temporal_weight"]).to(dev) if with_w else None
    stab = None if m is None else torch.tensor([m], dtype=torch.float32, device=dev)
    ctx, he, saved = m2.fwd_blend(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], stability=stab,
                                  temporal_weight=w)
    g = m2.bwd_blend(t["h_history"], t["h_s2"], saved, dhe, D, temporal_weight=w)
    torch.cuda.synchronize()
    got = {"context": ctx, "h_enriched": he, **g}
    if rows is not None:
        idx = torch.from_numpy(rows).to(dev)
        for k in ("context", "h_enriched", "d_context"):
            got[k] = got[k].index_select(0, idx)
    return {k: v.cpu().numpy() for k, v in got.items()}


def check_blend(inputs, extras, m, with_w, rows=None):
    got = run_blend(inputs, extras, m, with_w, rows)
    w = extras["temporal_weight"] if with_w else None
    f, he, bb, b = orc.fwd_bwd_blend(inputs, 1.0 if m is None else m, w, extras["d_h_enriched"])
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    assert_elementwise(got["context"], sel(f.context), "context")
    assert_elementwise(got["h_enriched"], sel(he), "h_enriched")
    assert_elementwise(got["d_context"], sel(bb.d_context), "d_context")
    for name in ("dW_A", "dW_B", "dW_C"):
        assert_l1(got[name], getattr(b, name), name)
    assert_l1(got["d_temporal_weight"], bb.d_temporal_weight, "d_temporal_weight")
    return f


@pytest.mark.parametrize("B,K,SH2,D", EDGE_SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("m,with_w", [(None, False), (0.9, True)], ids=["plain", "stab0.9_w"])
def test_blend_edge_shapes(B, K, SH2, D, m, with_w):
    seed = B * 5 + K
    check_blend(make_inputs(B, K, SH2, D, seed=seed), blend_extras(B, SH2, seed), m, with_w)


# The blend fused into the wide-trunk forms at one state group: a two-block
# full pass (257 pairs of blocks) and a two-block replay after a one-block
# summary pass.
@pytest.mark.parametrize("B,K,SH2,D", [(8200, 2, 320, 16), (20, 96, 384, 16)], ids=lambda v: str(v))
def test_blend_launch_forms(B, K, SH2, D):
    seed = B + K + 11
    check_blend(make_inputs(B, K, SH2, D, seed=seed, gate_bias=2.0 if K >= 32 else 0.0),
                blend_extras(B, SH2, seed), 0.9, True)


@pytest.mark.parametrize("name,m", [("tiny", 1.1), ("mid", 0.8), ("pages_shape", 0.95)])
def test_blend_workloads(name, m):
    inputs = workload_inputs(name)
    B, _, SH2 = inputs["h_history"].shape
    check_blend(inputs, blend_extras(B, SH2, 7), m, True)


@pytest.mark.parametrize("name", ["long_history", "wide_state"])
def test_blend_large_sampled_rows(name):
    """Full-size launches; per-sample outputs compared on 512 sampled rows, weight gradients in full."""
    inputs = workload_inputs(name)
    B, _, SH2 = inputs["h_history"].shape
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(B - 16, B), rng.choice(B, 480, replace=False)]))
    f = check_blend(inputs, blend_extras(B, SH2, 8), 0.98, True, rows)
    if name == "long_history":
        # the multiplier shortens the memory: mean effective gate m * sigma(a)
        assert 0.78 < float(np.mean(0.98 * f.g)) < 0.93


def test_blend_plain_matches_scan_path_bitwise():
    """No multiplier and no weights: the blend's forward equals mamba2_scan_fwd bit for bit, and its
    backward equals mamba2_scan_bwd run on the d_context it produced."""
    inputs = make_inputs(300, 12, 256, 16, seed=31)
    extras = blend_extras(300, 256, 31)
    t = _to_dev(inputs)
    dhe = torch.from_numpy(extras["d_h_enriched"]).to(t["h_s2"].device)
    ctx0, saved0 = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    ctx1, he, saved1 = m2.fwd_blend(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    g1 = m2.bwd_blend(t["h_history"], t["h_s2"], saved1, dhe, 16)
    g0 = m2.bwd(t["h_history"], t["h_s2"], saved0, g1["d_context"])
    torch.cuda.synchronize()
    assert torch.equal(ctx0, ctx1) and torch.equal(saved0, saved1)
    for n in ("dW_A", "dW_B", "dW_C"):
        assert torch.equal(g0[n], g1[n]), n
    # stability 1.0 given explicitly: still the same bits
    one = torch.ones(1, device=ctx0.device)
    ctx2, _, saved2 = m2.fwd_blend(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], stability=one)
    torch.cuda.synchronize()
    assert torch.equal(ctx0, ctx2) and torch.equal(saved0, saved2)


def test_blend_optional_outputs_and_determinism():
    inputs = make_inputs(200, 9, 192, 32, seed=41)
    extras = blend_extras(200, 192, 41)
    t = _to_dev(inputs)
    dev = t["h_s2"].device
    dhe = torch.from_numpy(extras["d_h_enriched"]).to(dev)
    w = torch.from_numpy(extras["temporal_weight"]).to(dev)
    stab = torch.tensor([0.85], device=dev)
    ctx, none, saved = m2.fwd_blend(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], stability=stab,
                                    temporal_weight=w, want_h_enriched=False)
    assert none is None
    a = m2.bwd_blend(t["h_history"], t["h_s2"], saved, dhe, 32, temporal_weight=w)
    b = m2.bwd_blend(t["h_history"], t["h_s2"], saved, dhe, 32, temporal_weight=w, want_d_temporal_weight=False)
    torch.cuda.synchronize()
    assert b.get("d_temporal_weight") is None
    for n in ("dW_A", "dW_B", "dW_C", "d_context"):
        assert torch.equal(a[n], b[n]), n
    f, _, bb, g = orc.fwd_bwd_blend(inputs, 0.85, extras["temporal_weight"], extras["d_h_enriched"])
    assert_elementwise(ctx.cpu().numpy(), f.context, "context")
    assert_l1(a["d_temporal_weight"].cpu().numpy(), bb.d_temporal_weight, "d_temporal_weight")


def test_blend_binding_errors():
    inputs = make_inputs(20, 4, 128, 16, seed=3)
    t = _to_dev(inputs)
    dev = t["h_s2"].device
    ctx, he, saved = m2.fwd_blend(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    dhe = torch.zeros((20, 128), device=dev)
    ws = torch.empty(m2.workspace_bytes(20, 4, 128, 16) // 4, device=dev)  # the scan's size: too small
    with pytest.raises(m2.Mamba2ScanError):
        m2.bwd_blend(t["h_history"], t["h_s2"], saved, dhe, 16, workspace=ws)
    with pytest.raises(ValueError):
        m2.fwd_blend(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"],
                     temporal_weight=torch.ones(127, device=dev))
