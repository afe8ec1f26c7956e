"""mamba2_scan_bwd_noalloc (the backward for callers that cannot allocate)
against mamba2_scan_bwd, through the C-ABI, on an MI355X.

Both run the same kernels; the no-alloc call keeps its split-K slices in the
library's own per-device buffer instead of a caller workspace, so the weight
gradients and the optional d_a, d_b, d_c must agree bit for bit, and with the
oracle within the path's tolerances.  Two calls in a row share the buffer:
the second, smaller one must not see the first one's slices.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import bwd_mamba2_scan_amd as m2
from oracle import mamba2_oracle as orc
from tests.inputs import make_inputs
from tests.test_parity_gpu import _to_dev, assert_elementwise, assert_l1

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(t, saved, B, K, SH2, D):
    dev = saved.device
    out = {k: torch.full((SH2, D), float("nan"), device=dev) for k in ("dW_A", "dW_B", "dW_C")}
    out["d_a"] = torch.full((B, K, D), float("nan"), device=dev)
    out["d_b"] = torch.full((B, K, D), float("nan"), device=dev)
    out["d_c"] = torch.full((B, D), float("nan"), device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = m2.lib().mamba2_scan_bwd_noalloc(
        B, K, SH2, D, _p(t["h_history"]), _p(t["h_s2"]), _p(saved), saved.numel() * 4, _p(t["d_context"]),
        _p(out["dW_A"]), _p(out["dW_B"]), _p(out["dW_C"]), _p(out["d_a"]), _p(out["d_b"]), _p(out["d_c"]), stream)
    assert st == m2.OK, m2.strerror(st)
    return out


# the first shape needs nearly the whole buffer (3.2 MiB of slices); the second is smaller
SHAPES = [(1000, 20, 448, 64), (33, 9, 256, 16)]


def test_noalloc_matches_bwd_on_two_calls():
    print("no-alloc backward: shapes", SHAPES, flush=True)
    for B, K, SH2, D in SHAPES:
        inputs = make_inputs(B, K, SH2, D, seed=B + K + 2)
        t = _to_dev(inputs)
        _, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
        ref = m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"], debug=True)
        got = _noalloc(t, saved, B, K, SH2, D)
        torch.cuda.synchronize()
        for k in ("dW_A", "dW_B", "dW_C", "d_a", "d_b", "d_c"):
            assert torch.equal(got[k], ref[k]), (B, K, SH2, D, k)
        _, b = orc.fwd_bwd(inputs)
        for k in ("dW_A", "dW_B", "dW_C"):
            assert_l1(got[k].cpu().numpy(), getattr(b, k), k)
        for k in ("d_a", "d_b", "d_c"):
            assert_elementwise(got[k].cpu().numpy(), getattr(b, k), k)
