"""The oracle against its pins, and the pins against planted mistakes (CPU only)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import mamba2_oracle as orc
from tests import pins


@pytest.mark.parametrize("check", pins.ALL_PINS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(orc)


# ------------------------------------------------------------------ mutations
# Each mutant plants one plausible mistake in the oracle (on the CPU, through
# monkeypatch).  At least one pin must fail for every mutant; otherwise the
# pins would not notice that mistake.
def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _scan_fwd_time_reversed(a, bb, m=1.0):
    a, bb = _f64(a), _f64(bb)
    B, K, D = a.shape
    g = orc.logistic(a)
    x = np.zeros((B, K + 1, D))
    for step, t in enumerate(range(K - 1, -1, -1)):
        x[:, step + 1] = m * g[:, t] * x[:, step] + bb[:, t]
    return g, x


def _scan_fwd_x0_one(a, bb, m=1.0):
    a, bb = _f64(a), _f64(bb)
    B, K, D = a.shape
    g = orc.logistic(a)
    x = np.ones((B, K + 1, D))
    for t in range(K):
        x[:, t + 1] = m * g[:, t] * x[:, t] + bb[:, t]
    return g, x


def _scan_fwd_stability_on_input(a, bb, m=1.0):
    # plausible mistake: the multiplier scales the new input instead of the gate
    a, bb = _f64(a), _f64(bb)
    B, K, D = a.shape
    g = orc.logistic(a)
    x = np.zeros((B, K + 1, D))
    for t in range(K):
        x[:, t + 1] = g[:, t] * x[:, t] + m * bb[:, t]
    return g, x


def _make_scan_bwd(x_index_shift=0, dx_k_times_c=True, sig_prime=True, carry_gate=True, m_in_d_a=True,
                   m_in_carry=True):
    def scan_backward(g, x, c, d_context, m=1.0):
        g, x, d_context = _f64(g), _f64(x), _f64(d_context)
        B, K, D = g.shape
        dx = d_context * _f64(c) if dx_k_times_c else d_context.copy()
        d_c = d_context * x[:, K]
        d_a = np.empty((B, K, D))
        d_b = np.empty((B, K, D))
        for t in range(K - 1, -1, -1):
            gt = g[:, t]
            d_b[:, t] = dx
            sp = gt * (1.0 - gt) if sig_prime else gt
            d_a[:, t] = dx * x[:, t + x_index_shift] * sp * (m if m_in_d_a else 1.0)
            dx = dx * (gt if carry_gate else (1.0 - gt)) * (m if m_in_carry else 1.0)
        return d_a, d_b, d_c
    return scan_backward


def _backward_dwc_from_dcontext(fwd, h_history, h_s2, d_context):
    b = _ORIG_BACKWARD(fwd, h_history, h_s2, d_context)
    b.dW_C = _f64(h_s2).T @ _f64(d_context)
    return b


def _backward_swapped_planes(fwd, h_history, h_s2, d_context):
    b = _ORIG_BACKWARD(fwd, h_history, h_s2, d_context)
    b.dW_A, b.dW_B = b.dW_B, b.dW_A
    return b


def _forward_sum_readout(h_history, h_s2, W_A, W_B, W_C, stability=1.0):
    f = _ORIG_FORWARD(h_history, h_s2, W_A, W_B, W_C, stability)
    f.context = f.c + f.x[:, -1]
    return f


def _blend_without_mean(context, h_s2, temporal_weight=None):
    D = _f64(context).shape[1]
    return _ORIG_BLEND(context, h_s2, temporal_weight) * 1.0 + (D - 1) * (
        _ORIG_BLEND(context, h_s2, temporal_weight) - _f64(h_s2))


def _blend_bwd_first_state_only(d_h_enriched, context, temporal_weight=None):
    r = _ORIG_BLEND_BWD(d_h_enriched, context, temporal_weight)
    r.d_context[:, 1:] = 0.0
    return r


def _blend_bwd_weight_without_mean(d_h_enriched, context, temporal_weight=None):
    r = _ORIG_BLEND_BWD(d_h_enriched, context, temporal_weight)
    r.d_temporal_weight = r.d_temporal_weight * _f64(context).shape[1]
    return r


def _blend_bwd_ignores_weight(d_h_enriched, context, temporal_weight=None):
    # plausible mistake: d_context taken as if every temporal weight were 1
    r = _ORIG_BLEND_BWD(d_h_enriched, context, None)
    w_r = _ORIG_BLEND_BWD(d_h_enriched, context, temporal_weight)
    r.d_temporal_weight = w_r.d_temporal_weight
    return r


def _input_grads_wrong_weight(bwd, W_A, W_B, W_C):
    g = _ORIG_INPUT_GRADS(bwd, W_A, W_B, W_C)
    B, K, D = bwd.d_a.shape
    if g.d_h_history.shape[2] == D:  # only well-defined for square weights
        return g
    # plausible mistake: d_b multiplied by W_A instead of W_B
    dH = bwd.d_a.reshape(B * K, D) @ _f64(W_A).T + bwd.d_b.reshape(B * K, D) @ _f64(W_A).T
    g.d_h_history = dH.reshape(B, K, -1)
    return g


_ORIG_BACKWARD = orc.backward
_ORIG_FORWARD = orc.forward
_ORIG_INPUT_GRADS = orc.input_grads
_ORIG_BLEND = orc.blend
_ORIG_BLEND_BWD = orc.blend_backward

MUTANTS = {
    "gate_sign_flipped": ("logistic", lambda a: 1.0 / (1.0 + np.exp(_f64(a)))),
    "projection_columns_reversed": ("project", lambda rows, W: _f64(rows) @ _f64(W)[:, ::-1]),
    "projection_drops_first_feature": ("project", lambda rows, W: _f64(rows)[:, 1:] @ _f64(W)[1:]),
    "scan_time_reversed": ("scan_forward", _scan_fwd_time_reversed),
    "scan_initial_state_one": ("scan_forward", _scan_fwd_x0_one),
    "bwd_uses_next_state": ("scan_backward", _make_scan_bwd(x_index_shift=1)),
    "bwd_drops_c_in_dx_K": ("scan_backward", _make_scan_bwd(dx_k_times_c=False)),
    "bwd_drops_sigmoid_derivative": ("scan_backward", _make_scan_bwd(sig_prime=False)),
    "bwd_carries_one_minus_gate": ("scan_backward", _make_scan_bwd(carry_gate=False)),
    "dWC_from_d_context": ("backward", _backward_dwc_from_dcontext),
    "dWA_dWB_swapped": ("backward", _backward_swapped_planes),
    "readout_added_not_multiplied": ("forward", _forward_sum_readout),
    "input_grad_uses_wrong_weight": ("input_grads", _input_grads_wrong_weight),
    "stability_scales_input": ("scan_forward", _scan_fwd_stability_on_input),
    "stability_missing_in_d_a": ("scan_backward", _make_scan_bwd(m_in_d_a=False)),
    "stability_missing_in_carry": ("scan_backward", _make_scan_bwd(m_in_carry=False)),
    "blend_sums_instead_of_mean": ("blend", _blend_without_mean),
    "blend_d_context_first_state_only": ("blend_backward", _blend_bwd_first_state_only),
    "blend_d_weight_without_mean": ("blend_backward", _blend_bwd_weight_without_mean),
    "blend_d_context_ignores_weight": ("blend_backward", _blend_bwd_ignores_weight),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    failed = []
    for check in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                check(orc)
        except Exception:  # an assertion, or a shape/overflow error the mistake causes
            failed.append(check.__name__)
    assert failed, f"no pin notices mutant {name}"


def test_oracle_matches_frozen_golden():
    """Regression freeze: the oracle still reproduces tests/golden/oracle_tiny.json."""
    import json
    import os

    from tests.inputs import make_inputs

    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")
    with open(path) as fh:
        gold = json.load(fh)
    f, b = orc.fwd_bwd(make_inputs(**gold["shape"]))
    np.testing.assert_allclose(f.context, np.array(gold["context"]), rtol=1e-12, atol=1e-14)
    for name in ("dW_A", "dW_B", "dW_C"):
        np.testing.assert_allclose(getattr(b, name), np.array(gold[name]), rtol=1e-12, atol=1e-14)
