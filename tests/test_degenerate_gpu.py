"""Degenerate inputs and concurrent calls, on an MI355X.

* d_context = 0: every gradient of L = sum d_context * context is exactly
  zero (the weight gradients, the input gradients, d_a, d_b, d_c).
* W_A = W_B = W_C = 0: a = b = c = 0, so x stays 0, context is exactly zero
  and so is every gradient (d_b = d_context * c * prod g = 0, d_a carries x).
* A NaN in one history entry: the forward keeps it in its own sample (that
  row of context is NaN, every other row matches the oracle), and the NaN
  pattern of every output matches the oracle's, which propagates it the
  same way (samples are independent in the forward; the weight gradients
  sum over all samples).
* Two streams running independent batches at once give the same bits as
  the same calls one after the other (the library keeps no state between
  calls).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_mamba2_scan_amd as m2
from oracle import mamba2_oracle as orc
from tests.inputs import make_inputs
from tests.test_parity_gpu import _to_dev, assert_elementwise, assert_l1

pytestmark = pytest.mark.gpu

SHAPES = [(33, 9, 256, 16), (40, 8, 320, 64), (17, 3, 128, 32)]


def _all(t, K, debug=True):
    ctx, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    g = m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"], debug=debug)
    dH, dhs2 = m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, t["d_context"], K)
    full = m2.bwd_full(t["h_history"], t["h_s2"], saved, t["d_context"], t["W_A"], t["W_B"], t["W_C"])
    torch.cuda.synchronize()
    out = {"context": ctx, "d_h_history": dH, "d_h_s2": dhs2, **g}
    out.update({f"full_{k}": v for k, v in full.items()})
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("B,K,SH2,D", SHAPES, ids=lambda v: str(v))
def test_zero_upstream_gradient(B, K, SH2, D):
    inputs = make_inputs(B, K, SH2, D, seed=B + K)
    inputs["d_context"] = np.zeros_like(inputs["d_context"])
    got = _all(_to_dev(inputs), K)
    for k, v in got.items():
        if k != "context":
            assert np.all(v == 0.0), f"{k}: {np.count_nonzero(v)} nonzero values"
    f = orc.forward(inputs["h_history"], inputs["h_s2"], inputs["W_A"], inputs["W_B"], inputs["W_C"])
    assert_elementwise(got["context"], f.context, "context")


@pytest.mark.parametrize("B,K,SH2,D", SHAPES, ids=lambda v: str(v))
def test_zero_weights(B, K, SH2, D):
    inputs = make_inputs(B, K, SH2, D, seed=B + 2 * K)
    for k in ("W_A", "W_B", "W_C"):
        inputs[k] = np.zeros_like(inputs[k])
    got = _all(_to_dev(inputs), K)
    for k, v in got.items():
        assert np.all(v == 0.0), f"{k}: {np.count_nonzero(v)} nonzero values"


@pytest.mark.parametrize("B,K,SH2,D", SHAPES, ids=lambda v: str(v))
def test_nan_stays_in_its_sample(B, K, SH2, D):
    inputs = make_inputs(B, K, SH2, D, seed=B + 3 * K)
    bad = B // 2
    inputs["h_history"][bad, K // 2, SH2 // 3] = np.nan
    got = _all(_to_dev(inputs), K)
    with np.errstate(invalid="ignore", over="ignore"):
        f, b = orc.fwd_bwd(inputs)
        ig = orc.input_grads(b, inputs["W_A"], inputs["W_B"], inputs["W_C"])
    ctx = got["context"]
    assert np.all(np.isnan(ctx[bad])), "the sample with the NaN keeps it in every state"
    keep = np.arange(B) != bad
    assert_elementwise(ctx[keep], f.context[keep], "context of the other samples")
    ref = {"dW_A": b.dW_A, "dW_B": b.dW_B, "dW_C": b.dW_C, "d_a": b.d_a.reshape(B * K, D),
           "d_b": b.d_b.reshape(B * K, D), "d_c": b.d_c, "d_h_history": ig.d_h_history, "d_h_s2": ig.d_h_s2}
    for k, r in ref.items():
        for name in (k, f"full_{k}"):
            if name not in got:
                continue
            v = got[name].reshape(r.shape)
            assert np.array_equal(np.isnan(v), np.isnan(r)), f"{name}: NaN pattern differs from the oracle's"
            fin = ~np.isnan(r)
            base = name[len("full_"):] if name.startswith("full_") else name
            if fin.any() and base.startswith("d_"):
                assert_elementwise(v[fin], r[fin], f"{name} (finite entries)")


def test_two_streams_match_sequential():
    sets = [make_inputs(1000, 9, 256, 16, seed=s) for s in (41, 42)]
    ts = [_to_dev(x) for x in sets]
    seq = [_all(t, 9, debug=False) for t in ts]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    torch.cuda.synchronize()
    for i, (t, s) in enumerate(zip(ts, streams)):
        with torch.cuda.stream(s):
            ctx, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], stream=s)
            g = m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"], stream=s)
            full = m2.bwd_full(t["h_history"], t["h_s2"], saved, t["d_context"], t["W_A"], t["W_B"], t["W_C"],
                               stream=s)
            outs[i] = (ctx, g, full)
    torch.cuda.synchronize()
    for i in range(2):
        ctx, g, full = outs[i]
        assert np.array_equal(ctx.cpu().numpy(), seq[i]["context"]), "context"
        for k in ("dW_A", "dW_B", "dW_C"):
            assert np.array_equal(g[k].cpu().numpy(), seq[i][k]), k
        for k in ("dW_A", "dW_B", "dW_C", "d_h_history", "d_h_s2"):
            assert np.array_equal(full[k].cpu().numpy(), seq[i][f"full_{k}"]), f"full {k}"
    # and the concurrent results still hold against the oracle
    f, b = orc.fwd_bwd(sets[0])
    assert_elementwise(outs[0][0].cpu().numpy(), f.context, "context")
    for k in ("dW_A", "dW_B", "dW_C"):
        assert_l1(outs[0][1][k].cpu().numpy(), getattr(b, k), k)
