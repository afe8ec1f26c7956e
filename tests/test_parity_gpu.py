"""Parity of the HIP path against the CPU oracle, on an MI355X.

Tolerances (the accuracy the path is held to):
  * outputs (context, and d_a, d_b, d_c when requested): elementwise
    |gpu - ref| <= 1e-4 * (1 + |ref|)
  * weight gradients: sum|gpu - ref| / sum|ref| <= 1e-3 per matrix.
The GPU accumulates in fp32 (the backward's products are fp32 MFMAs, the
forward's are bf16 MFMAs on operands split exactly into three bf16 terms); the
oracle computes in fp64.  test_fp32_class_accuracy holds the path to the
accuracy of fp32 arithmetic, well inside the tolerances above.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_mamba2_scan_amd as m2
from oracle import mamba2_oracle as orc
from tests.inputs import WORKLOADS, make_inputs, workload_inputs
from tests.shapes import EDGE_SHAPES, FORM_SHAPES, FP32_WORKLOADS, LONG_FEW_SHAPES, gate_bias

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-4
DW_TOL = 1e-3


def _dev():
    assert torch.cuda.is_available(), "no GPU visible"
    return torch.device("cuda:0")


def _to_dev(inputs):
    dev = _dev()
    return {k: torch.from_numpy(v).to(dev) for k, v in inputs.items()}


def run_gpu(t, debug=False):
    ctx, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    g = m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"], debug=debug)
    torch.cuda.synchronize()
    out = {"context": ctx.cpu().numpy()}
    out.update({k: v.cpu().numpy() for k, v in g.items()})
    return out


def assert_elementwise(gpu, ref, name, tol=OUT_TOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    err = np.abs(gpu - ref)
    bound = tol * (1.0 + np.abs(ref))
    worst = int(np.argmax(err / bound))
    assert np.all(err <= bound), (
        f"{name}: {int(np.sum(err > bound))} of {err.size} elements out of tolerance; worst at flat index "
        f"{worst}: gpu={gpu.flat[worst]!r} ref={ref.flat[worst]!r}")


def assert_l1(gpu, ref, name, tol=DW_TOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    den = float(np.sum(np.abs(ref)))
    rel = float(np.sum(np.abs(gpu - ref))) / den if den > 0 else float(np.sum(np.abs(gpu)))
    assert rel <= tol, f"{name}: L1 relative error {rel:.3e} > {tol:.1e}"


def check_against_oracle(inputs, debug=True):
    t = _to_dev(inputs)
    got = run_gpu(t, debug=debug)
    f, b = orc.fwd_bwd(inputs)
    assert_elementwise(got["context"], f.context, "context")
    for name in ("dW_A", "dW_B", "dW_C"):
        assert_l1(got[name], getattr(b, name), name)
    if debug:
        assert_elementwise(got["d_a"], b.d_a, "d_a")
        assert_elementwise(got["d_b"], b.d_b, "d_b")
        assert_elementwise(got["d_c"], b.d_c, "d_c")
    return got, f, b


@pytest.mark.parametrize("B,K,SH2,D", EDGE_SHAPES, ids=lambda v: str(v))
def test_edge_shapes(B, K, SH2, D):
    check_against_oracle(make_inputs(B, K, SH2, D, seed=B * 7 + K))


@pytest.mark.parametrize("name", FP32_WORKLOADS[:3])
def test_workload_full(name):
    check_against_oracle(workload_inputs(name), debug=(name != "pages_shape"))


@pytest.mark.parametrize("name", FP32_WORKLOADS[3:])
def test_workload_large(name):
    got, f, _ = check_against_oracle(workload_inputs(name), debug=False)
    if name in ("long_history", "long_few"):
        # the +2 logit shift gives long-memory gates
        assert 0.8 < float(np.mean(f.g)) < 0.95


def test_saturated_and_extreme_logits():
    """Gates pinned at 0 (states 0-3) and 1 (states 4-7) with |a| ~ 100, the
    other states ordinary: finite results and oracle parity.  In the pinned
    states sigma'(a) ~ e^-100 underflows fp32, so their dW_A columns are ~0 on
    both sides and are checked by absolute size instead."""
    inp = make_inputs(48, 6, 128, 16, seed=77)
    inp["h_history"][:, :, 0] = 1.0
    inp["W_A"][0, :4] = -100.0
    inp["W_A"][0, 4:8] = 100.0
    got, f, b = check_against_oracle(inp)
    assert np.max(np.abs(b.dW_A[:, :8])) < 1e-30
    assert np.max(np.abs(got["dW_A"][:, :8])) < 1e-30
    assert np.all(f.g[:, :, :4] < 1e-40) and np.all(f.g[:, :, 4:8] == 1.0)


def test_bitwise_determinism():
    """Same inputs, same shape -> identical bits for context and every dW."""
    t = _to_dev(workload_inputs("mid"))
    r1 = run_gpu(t)
    r2 = run_gpu(t)
    for k in ("context", "dW_A", "dW_B", "dW_C"):
        assert np.array_equal(r1[k].view(np.uint32), r2[k].view(np.uint32)), k


def test_split_phase_matches_bwd():
    """bwd_partials + bwd_reduce gives the same bits as bwd."""
    inp = make_inputs(200, 8, 256, 32, seed=5)
    t = _to_dev(inp)
    B, K, SH2 = inp["h_history"].shape
    D = inp["W_A"].shape[1]
    ctx, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    one = m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"])
    ws = m2.alloc_workspace(B, K, SH2, D, t["h_history"].device)
    m2.bwd_partials(t["h_history"], t["h_s2"], saved, t["d_context"], ws)
    outs = [torch.empty((SH2, D), device=ws.device) for _ in range(3)]
    m2.bwd_reduce(B, K, SH2, D, ws, *outs)
    torch.cuda.synchronize()
    for o, k in zip(outs, ("dW_A", "dW_B", "dW_C")):
        assert torch.equal(o, one[k]), k


def test_batch_split_additivity():
    """dW(all samples) = dW(first part) + dW(rest); context rows do not depend on the split."""
    inp = make_inputs(160, 8, 256, 16, seed=9)
    t = _to_dev(inp)
    full = run_gpu(t)
    cut = 70
    parts = []
    for sl in (slice(0, cut), slice(cut, None)):
        tp = {k: (v[sl].contiguous() if k in ("h_history", "h_s2", "d_context") else v) for k, v in t.items()}
        parts.append(run_gpu(tp))
    np.testing.assert_allclose(np.concatenate([parts[0]["context"], parts[1]["context"]]), full["context"],
                               rtol=0, atol=0)
    for k in ("dW_A", "dW_B", "dW_C"):
        assert_l1(parts[0][k].astype(np.float64) + parts[1][k], full[k].astype(np.float64), k, tol=1e-5)


def test_outputs_overwritten_not_accumulated():
    """Pre-filled output buffers are overwritten (the pages' bias-grad reduce that accumulates is not followed)."""
    inp = make_inputs(32, 4, 128, 16, seed=3)
    t = _to_dev(inp)
    B, K, SH2 = inp["h_history"].shape
    D = 16
    ctx = torch.full((B, D), 123.0, device=t["h_s2"].device)
    ctx, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], context=ctx)
    out = {k: torch.full((SH2, D), -7.0, device=ctx.device) for k in ("dW_A", "dW_B", "dW_C")}
    m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"], out=out)
    torch.cuda.synchronize()
    f, b = orc.fwd_bwd(inp)
    assert_elementwise(ctx.cpu().numpy(), f.context, "context")
    for k in ("dW_A", "dW_B", "dW_C"):
        assert_l1(out[k].cpu().numpy(), getattr(b, k), k)


def test_binding_rejects_bad_arguments():
    dev = _dev()
    h = torch.zeros((4, 2, 64), device=dev)
    hs = torch.zeros((4, 64), device=dev)
    w = torch.zeros((64, 16), device=dev)
    with pytest.raises(TypeError):
        m2.fwd(h.double(), hs, w, w, w)
    with pytest.raises(ValueError):
        m2.fwd(h, hs[:, :32].contiguous(), w, w, w)
    with pytest.raises(ValueError):
        m2.fwd(h, hs, w.t(), w, w)
    w8 = torch.zeros((64, 8), device=dev)
    with pytest.raises(ValueError):
        m2.fwd(h, hs, w8, w8, w8)
    ctx, saved = m2.fwd(h, hs, w, w, w)
    with pytest.raises(m2.Mamba2ScanError):
        m2.bwd(h, hs, saved[:-1], torch.zeros((4, 16), device=dev))
    torch.cuda.synchronize()


def test_workloads_table_matches_pages_shape():
    w = WORKLOADS["pages_shape"]
    assert (w.B, w.K, w.SH2, w.D) == (8192, 8, 256, 16)


@pytest.mark.parametrize("B,K,SH2,D,bf16", [(300, 8, 256, 32, False), (17, 160, 192, 16, False),
                                             (300, 8, 256, 16, True), (17, 160, 192, 16, True)],
                         ids=lambda v: str(v))
def test_graph_replays_match_eager(B, K, SH2, D, bf16):
    """fwd + bwd captured in a HIP graph and replayed several times, with eager
    work and synchronisation between replays, give the eager bits every time
    (the library enqueues no memset and allocates nothing, so it is capturable).
    The second shape takes the chunked forward (summary, carry, replay)."""
    inp = make_inputs(B, K, SH2, D, seed=21, gate_bias=2.0 if K > 8 else 0.0)
    t = _to_dev(inp)
    if bf16:
        for k in ("h_history", "h_s2"):
            t[k] = t[k].to(torch.bfloat16)
    dev = t["h_history"].device

    ctx = torch.empty((B, D), device=dev)
    saved = m2.alloc_saved(B, K, SH2, D, dev)
    ws = m2.alloc_workspace(B, K, SH2, D, dev)
    out = {k: torch.empty((SH2, D), device=dev) for k in ("dW_A", "dW_B", "dW_C")}
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], context=ctx, saved=saved)
        m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"], workspace=ws, out=out)
    torch.cuda.synchronize()
    eager = {"context": ctx.cpu().numpy().copy()}
    eager.update({k: v.cpu().numpy().copy() for k, v in out.items()})
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], context=ctx, saved=saved)
        m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"], workspace=ws, out=out)
    for rep in range(4):
        # scribble over the outputs and the saved terms eagerly, then replay
        ctx.fill_(float("nan"))
        saved.fill_(float("nan"))
        for v in out.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(ctx.cpu().numpy().view(np.uint32), eager["context"].view(np.uint32)), rep
        for k in ("dW_A", "dW_B", "dW_C"):
            assert np.array_equal(out[k].cpu().numpy().view(np.uint32), eager[k].view(np.uint32)), (rep, k)


@pytest.mark.parametrize("B,K,SH2,D", LONG_FEW_SHAPES, ids=lambda v: str(v))
def test_chunked_history(B, K, SH2, D):
    inputs = make_inputs(B, K, SH2, D, seed=B + K, gate_bias=2.0)
    got, f, _ = check_against_oracle(inputs, debug=True)
    assert 0.8 < float(np.mean(f.g)) < 0.95  # long memory: the carry spans many chunks


@pytest.mark.parametrize("B,K,SH2,D", FORM_SHAPES, ids=lambda v: str(v))
def test_launch_forms(B, K, SH2, D):
    """The forward launch forms of wide trunks (two sample blocks per work-group,
    one-block summary passes, two-block replays), each against the oracle."""
    inputs = make_inputs(B, K, SH2, D, seed=B + 3 * K + SH2, gate_bias=gate_bias(K))
    check_against_oracle(inputs, debug=True)


def test_chunked_history_blend_and_input_grads():
    """The chunked forward with the stability multiplier feeds the blend backward and the input gradients."""
    from tests.inputs import blend_extras
    inputs = make_inputs(32, 512, 128, 16, seed=9, gate_bias=2.0)
    extras = blend_extras(32, 128, 9)
    t = _to_dev(inputs)
    dev = t["h_s2"].device
    stab = torch.tensor([0.97], device=dev)
    w = torch.from_numpy(extras["temporal_weight"]).to(dev)
    dhe = torch.from_numpy(extras["d_h_enriched"]).to(dev)
    ctx, he, saved = m2.fwd_blend(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], stability=stab,
                                  temporal_weight=w)
    g = m2.bwd_blend(t["h_history"], t["h_s2"], saved, dhe, 16, temporal_weight=w)
    dH, dhs2 = m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, g["d_context"], 512)
    torch.cuda.synchronize()
    f, he_ref, bb, b = orc.fwd_bwd_blend(inputs, 0.97, extras["temporal_weight"], extras["d_h_enriched"])
    assert_elementwise(ctx.cpu().numpy(), f.context, "context")
    assert_elementwise(he.cpu().numpy(), he_ref, "h_enriched")
    for name in ("dW_A", "dW_B", "dW_C"):
        assert_l1(g[name].cpu().numpy(), getattr(b, name), name)
    ig = orc.input_grads(b, inputs["W_A"], inputs["W_B"], inputs["W_C"])
    assert_elementwise(dH.cpu().numpy(), ig.d_h_history, "d_h_history")
    assert_elementwise(dhs2.cpu().numpy(), ig.d_h_s2, "d_h_s2")


# fp32-class accuracy: measured 3e-7 .. 8e-7 (elementwise err / (1 + |ref|))
# and 3e-7 .. 4e-7 (dW, L1) on an MI355X.  Products that kept only two bf16
# terms of an fp32 operand (2^-17 relative each) would give ~1e-5 here.
FP32_CLASS_OUT = 5e-6
FP32_CLASS_DW = 3e-6


@pytest.mark.parametrize("shape", [(300, 8, 256, 16), (300, 64, 256, 16), (64, 8, 512, 64), (40, 20, 192, 32)],
                         ids=["K8", "K64", "wide", "D32_rounds"])
def test_fp32_class_accuracy(shape):
    B, K, SH2, D = shape
    inp = make_inputs(B, K, SH2, D, seed=7)
    out = run_gpu(_to_dev(inp), debug=True)
    f, b = orc.fwd_bwd(inp)
    for name, gpu, ref in (("context", out["context"], f.context), ("d_a", out["d_a"], b.d_a),
                           ("d_b", out["d_b"], b.d_b), ("d_c", out["d_c"], b.d_c)):
        gpu = np.asarray(gpu, dtype=np.float64).reshape(ref.shape)
        worst = float(np.max(np.abs(gpu - ref) / (1.0 + np.abs(ref))))
        assert worst <= FP32_CLASS_OUT, f"{name}: {worst:.3e}"
    for name in ("dW_A", "dW_B", "dW_C"):
        ref = getattr(b, name)
        rel = float(np.sum(np.abs(np.asarray(out[name], np.float64) - ref)) / np.sum(np.abs(ref)))
        assert rel <= FP32_CLASS_DW, f"{name}: {rel:.3e}"
    # input gradients (bf16 split terms from D = 32 on, fp32 MFMAs at D = 16)
    t = _to_dev(inp)
    _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    dH, dhs2 = m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, t["d_context"], K)
    torch.cuda.synchronize()
    ig = orc.input_grads(b, inp["W_A"], inp["W_B"], inp["W_C"])
    for name, gpu, ref in (("d_h_history", dH, ig.d_h_history), ("d_h_s2", dhs2, ig.d_h_s2)):
        gpu = gpu.cpu().numpy().astype(np.float64)
        worst = float(np.max(np.abs(gpu - ref) / (1.0 + np.abs(ref))))
        assert worst <= FP32_CLASS_OUT, f"{name}: {worst:.3e}"
