"""Every forward launch form the dispatcher can choose is compared with the oracle.

CPU only: mamba2_scan_fwd_plan is host code (it reports the launches
mamba2_scan_fwd would enqueue without touching a device).  A launch form is
(SH2 / 16, kernel, sample blocks per work-group, pass): one compiled kernel
instantiation and the way it is driven.  The trunk precision (fp32 or bf16)
is a second instantiation of each, so each precision's shape list is checked
separately.

  * test_forms_closed: over a broad sweep of shapes the plan only ever
    chooses forms from FORMS (a new form added to the dispatcher fails here
    until it is listed), and every listed form is chosen by some shape.
  * test_gpu_shape_lists_reach_every_form: the shapes of the fp32 and bf16
    GPU parity tests (tests/shapes.py) together reach every form in FORMS.
"""
from __future__ import annotations

import itertools

import pytest

import bwd_mamba2_scan_amd as m2
from tests.shapes import BF16_FWD_SHAPES, FP32_FWD_SHAPES


def _expected_forms():
    """The forms of the dispatcher's rules: below SH2 = 320 a work-group holds
    one sample block; from SH2 = 320 on it holds two, except for full and
    summary passes whose two-block grid would leave CUs idle (then one); a
    chunked history adds the carry and a replay pass with the default count."""
    forms = set()
    for nkc in range(4, 33, 4):
        forms.add((nkc, "carry", 0, "carry"))
        if nkc < 20:
            for p in ("full", "summary", "replay"):
                forms.add((nkc, "fwd", 1, p))
        else:
            for blocks, p in ((1, "full"), (1, "summary"), (2, "full"), (2, "summary"), (2, "replay")):
                forms.add((nkc, "fwd", blocks, p))
    return forms


FORMS = _expected_forms()


def forms_of(B, K, SH2, D):
    return {(SH2 // 16, l["kernel"], l["sample_blocks"], l["pass"]) for l in m2.fwd_plan(B, K, SH2, D)}


def test_forms_closed():
    seen = set()
    Bs = (1, 15, 16, 17, 100, 255, 256, 511, 1000, 2033, 2048, 2050, 4081, 4096, 8176, 8177, 8192, 16384, 32768)
    Ks = (1, 8, 9, 31, 32, 40, 48, 64, 96, 100, 256, 1024, 2040, 8192)
    for B, K, SH2, D in itertools.product(Bs, Ks, range(64, 513, 64), (16, 32, 64)):
        f = forms_of(B, K, SH2, D)
        assert f <= FORMS, (B, K, SH2, D, f - FORMS)
        seen |= f
    assert seen == FORMS, sorted(FORMS - seen)


@pytest.mark.parametrize("name,shapes", [("fp32", FP32_FWD_SHAPES), ("bf16", BF16_FWD_SHAPES)])
def test_gpu_shape_lists_reach_every_form(name, shapes):
    reached = set().union(*(forms_of(*s) for s in shapes))
    assert reached == FORMS, f"{name}: forms no GPU parity test runs: {sorted(FORMS - reached)}"


def test_plan_shape_of_launches():
    # the pages' shape: one full pass, one work-group per 16-sample block
    (l,) = m2.fwd_plan(8192, 8, 256, 16)
    assert (l["kernel"], l["pass"], l["sample_blocks"], l["grid"], l["threads"]) == ("fwd", "full", 1, 512, 512)
    # a long history with few samples: summary, carry, replay over the same chunks
    ls = m2.fwd_plan(128, 2048, 256, 16)
    assert [l["pass"] for l in ls] == ["summary", "carry", "replay"]
    assert len({(l["chunks"], l["chunk_steps"]) for l in ls}) == 1
    c, steps = ls[0]["chunks"], ls[0]["chunk_steps"]
    assert c > 1 and steps % 16 == 0 and (c - 1) * steps < 2048 <= c * steps + steps
    # invalid or unsupported dimensions are refused, as by the forward itself
    with pytest.raises(m2.Mamba2ScanError):
        m2.fwd_plan(8, 8, 100, 16)
    with pytest.raises(m2.Mamba2ScanError):
        m2.fwd_plan(0, 8, 256, 16)
