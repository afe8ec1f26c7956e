"""Parity of the input gradients (mamba2_scan_bwd_input) against the CPU oracle.

d_h_history = d_a W_A^T + d_b W_B^T and d_h_s2 = d_c W_C^T, through the C-ABI.
Elementwise tolerance, as for the other outputs: |gpu - ref| <= 1e-4 (1 + |ref|).
The GPU computes in fp32 (the saved fp32 scan terms, fp32 MFMA); the oracle in fp64.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import bwd_mamba2_scan_amd as m2
from oracle import mamba2_oracle as orc
from tests.inputs import make_inputs, workload_inputs
from tests.shapes import EDGE_SHAPES, LONG_FEW_SHAPES
from tests.test_parity_gpu import _to_dev, assert_elementwise

pytestmark = pytest.mark.gpu


def gpu_input_grads(t, K, **kw):
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    dH, dhs2 = m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, t["d_context"], K, **kw)
    torch.cuda.synchronize()
    return dH, dhs2, saved


def oracle_input_grads(inputs, rows=None):
    """Oracle input gradients, optionally for a subset of samples only."""
    _, b = orc.fwd_bwd(inputs)
    if rows is not None:
        b = dataclasses.replace(b, d_a=b.d_a[rows], d_b=b.d_b[rows], d_c=b.d_c[rows])
    return orc.input_grads(b, inputs["W_A"], inputs["W_B"], inputs["W_C"])


@pytest.mark.parametrize("B,K,SH2,D", EDGE_SHAPES, ids=lambda v: str(v))
def test_input_grads_edge_shapes(B, K, SH2, D):
    inputs = make_inputs(B, K, SH2, D, seed=B * 7 + K + 1)
    dH, dhs2, _ = gpu_input_grads(_to_dev(inputs), K)
    ref = oracle_input_grads(inputs)
    assert_elementwise(dH.cpu().numpy(), ref.d_h_history, "d_h_history")
    assert_elementwise(dhs2.cpu().numpy(), ref.d_h_s2, "d_h_s2")


@pytest.mark.parametrize("name", ["tiny", "mid", "pages_shape"])
def test_input_grads_workloads(name):
    inputs = workload_inputs(name)
    K = inputs["h_history"].shape[1]
    dH, dhs2, _ = gpu_input_grads(_to_dev(inputs), K)
    ref = oracle_input_grads(inputs)
    assert_elementwise(dH.cpu().numpy(), ref.d_h_history, "d_h_history")
    assert_elementwise(dhs2.cpu().numpy(), ref.d_h_s2, "d_h_s2")


@pytest.mark.parametrize("B,K,SH2,D", LONG_FEW_SHAPES, ids=lambda v: str(v))
def test_input_grads_long_few(B, K, SH2, D):
    """Few samples, long histories: unit slices that start and end inside a block."""
    inputs = make_inputs(B, K, SH2, D, seed=B + K + 3, gate_bias=2.0)
    dH, dhs2, _ = gpu_input_grads(_to_dev(inputs), K)
    ref = oracle_input_grads(inputs)
    assert_elementwise(dH.cpu().numpy(), ref.d_h_history, "d_h_history")
    assert_elementwise(dhs2.cpu().numpy(), ref.d_h_s2, "d_h_s2")


def test_input_grads_several_batches():
    """A slice longer than one batch of units per wave: 50 samples, K = 6144,
    SH2 = 256 give 24,580 (block, step) units per column block, so the grid cap
    makes slices of 25 units per 4-wave work-group and a wave's seventh unit
    comes in a second, partial batch; every output against the oracle."""
    B, K, SH2, D = 50, 6144, 256, 16
    inputs = make_inputs(B, K, SH2, D, seed=23, gate_bias=2.0)
    dH, dhs2, _ = gpu_input_grads(_to_dev(inputs), K)
    ref = oracle_input_grads(inputs)
    assert_elementwise(dH.cpu().numpy(), ref.d_h_history, "d_h_history")
    assert_elementwise(dhs2.cpu().numpy(), ref.d_h_s2, "d_h_s2")


@pytest.mark.parametrize("name", ["long_history", "wide_state", "long_few"])
def test_input_grads_large_sampled(name):
    """Full-size launch; up to 512 samples (both ends, the middle, random) checked."""
    inputs = workload_inputs(name)
    B, K = inputs["h_history"].shape[:2]
    dH, dhs2, _ = gpu_input_grads(_to_dev(inputs), K)
    rng = np.random.default_rng(11)
    if B <= 512:
        rows = np.arange(B)
    else:
        rows = np.unique(np.concatenate([np.arange(16), np.arange(B - 16, B), B // 2 + np.arange(16),
                                         rng.choice(B, 464, replace=False)]))
    ref = oracle_input_grads(inputs, rows)
    idx = torch.from_numpy(rows).to(dH.device)
    assert_elementwise(dH.index_select(0, idx).cpu().numpy(), ref.d_h_history, "d_h_history")
    assert_elementwise(dhs2.index_select(0, idx).cpu().numpy(), ref.d_h_s2, "d_h_s2")


def test_input_grads_match_debug_terms():
    """The input gradients use the same d_a, d_b, d_c the weight-gradient backward forms."""
    inputs = make_inputs(300, 12, 256, 32, seed=21)
    t = _to_dev(inputs)
    dH, dhs2, saved = gpu_input_grads(t, 12)
    g = m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"], debug=True)
    B, K, D = g["d_a"].shape
    d_a = g["d_a"].double().reshape(B * K, D)
    d_b = g["d_b"].double().reshape(B * K, D)
    ref_h = (d_a @ t["W_A"].double().T + d_b @ t["W_B"].double().T).reshape(B, K, -1)
    ref_s = g["d_c"].double() @ t["W_C"].double().T
    assert_elementwise(dH.cpu().numpy(), ref_h.cpu().numpy(), "d_h_history vs debug terms", tol=1e-5)
    assert_elementwise(dhs2.cpu().numpy(), ref_s.cpu().numpy(), "d_h_s2 vs debug terms", tol=1e-5)


def test_input_grads_one_output_only_and_overwrite():
    inputs = make_inputs(77, 9, 192, 16, seed=5)
    t = _to_dev(inputs)
    dev = t["W_A"].device
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    ref = oracle_input_grads(inputs)
    nan_h = torch.full((77, 9, 192), float("nan"), device=dev)
    nan_s = torch.full((77, 192), float("nan"), device=dev)
    dH, none = m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, t["d_context"], 9, d_h_history=nan_h,
                            want=("h_history",))
    torch.cuda.synchronize()
    assert none is None
    assert_elementwise(dH.cpu().numpy(), ref.d_h_history, "d_h_history (alone, over NaN)")
    none, dhs2 = m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, t["d_context"], 9, d_h_s2=nan_s,
                              want=("h_s2",))
    torch.cuda.synchronize()
    assert none is None
    assert_elementwise(dhs2.cpu().numpy(), ref.d_h_s2, "d_h_s2 (alone, over NaN)")


def test_input_grads_bitwise_deterministic():
    inputs = make_inputs(1000, 8, 256, 16, seed=9)
    t = _to_dev(inputs)
    a_h, a_s, saved = gpu_input_grads(t, 8)
    b_h, b_s = m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, t["d_context"], 8)
    torch.cuda.synchronize()
    assert torch.equal(a_h, b_h) and torch.equal(a_s, b_s)


def test_input_grads_binding_errors():
    inputs = make_inputs(20, 4, 128, 16, seed=3)
    t = _to_dev(inputs)
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    with pytest.raises(m2.Mamba2ScanError):
        m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved[:-1], t["d_context"], 4)
    with pytest.raises(ValueError):
        m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, t["d_context"], 4,
                     d_h_history=torch.empty((20, 5, 128), device=saved.device))
