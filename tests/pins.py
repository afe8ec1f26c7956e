"""Pins that tie the CPU oracle to facts fixed by the pages and by mathematics.

The foxhunt pages print no worked numeric example for the Mamba2 scan, so every
pin here is a closed form, a special case that reduces to exact arithmetic or
to a library routine, an invariant, or brute force (central finite
differences) on tiny inputs.  Each check takes the oracle module as an argument
so that a test can plant a mistake in a copy of it and confirm a pin fails.

Each check raises AssertionError on failure.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
from scipy.special import expit


def _int_inputs(rng, B, K, SH2, D, w_lo=-4, w_hi=4):
    H = rng.integers(-3, 4, (B, K, SH2)).astype(np.float64)
    h_s2 = rng.integers(-3, 4, (B, SH2)).astype(np.float64)
    W_A = rng.integers(w_lo, w_hi + 1, (SH2, D)).astype(np.float64)
    W_B = rng.integers(w_lo, w_hi + 1, (SH2, D)).astype(np.float64)
    W_C = rng.integers(w_lo, w_hi + 1, (SH2, D)).astype(np.float64)
    return H, h_s2, W_A, W_B, W_C


def _real_inputs(rng, B, K, SH2, D, wa_scale=1.0):
    H = rng.standard_normal((B, K, SH2))
    h_s2 = rng.standard_normal((B, SH2))
    r = 1.0 / math.sqrt(SH2)
    W_A = rng.uniform(-wa_scale, wa_scale, (SH2, D))
    W_B = rng.uniform(-r, r, (SH2, D))
    W_C = rng.uniform(-r, r, (SH2, D))
    d_ctx = rng.standard_normal((B, D))
    return H, h_s2, W_A, W_B, W_C, d_ctx


def _dot_int(u, v):
    return sum(int(p) * int(q) for p, q in zip(u, v))


# ---------------------------------------------------------------- forward pins
def check_k1_closed_form(orc):
    """K = 1: x_1 = b_0 (x_0 = 0), so context = (h_s2 W_C) * (H_0 W_B) exactly.

    Integer inputs make every float64 operation exact; the expected value is
    computed with Python integers.  Non-square shapes catch a transposed W.
    """
    rng = np.random.default_rng(101)
    B, K, SH2, D = 3, 1, 5, 2
    H, h_s2, W_A, W_B, W_C = _int_inputs(rng, B, K, SH2, D)
    f = orc.forward(H, h_s2, W_A, W_B, W_C)
    for b in range(B):
        for s in range(D):
            c = _dot_int(h_s2[b], W_C[:, s])
            x1 = _dot_int(H[b, 0], W_B[:, s])
            assert f.context[b, s] == c * x1, (b, s, f.context[b, s], c * x1)


def check_half_gate_geometric(orc):
    """W_A = 0: every gate is exactly 1/2, so x_K = sum_t 2^-(K-1-t) b_t.

    Integer inputs keep the float64 result exact (dyadic rationals); the
    expected value uses Fractions.  The weights 2^-(K-1-t) fix the time order:
    the newest row t = K-1 has weight 1.  With all K rows equal to beta the sum
    is beta * (2 - 2^(1-K)) (K = 8: 1.9921875 * beta).
    """
    rng = np.random.default_rng(202)
    B, K, SH2, D = 3, 5, 6, 3
    H, h_s2, _, W_B, W_C = _int_inputs(rng, B, K, SH2, D)
    W_A = np.zeros((SH2, D))
    f = orc.forward(H, h_s2, W_A, W_B, W_C)
    assert np.all(f.g == 0.5)
    for b in range(B):
        for s in range(D):
            xk = sum(Fraction(_dot_int(H[b, t], W_B[:, s]), 2 ** (K - 1 - t)) for t in range(K))
            ctx = xk * _dot_int(h_s2[b], W_C[:, s])
            assert Fraction(f.context[b, s]) == ctx, (b, s)

    # equal rows: geometric closed form
    K = 8
    row = rng.integers(-3, 4, (1, 1, SH2)).astype(np.float64)
    Hs = np.repeat(row, K, axis=1)
    hs2 = np.ones((1, SH2))
    f = orc.forward(Hs, hs2, np.zeros((SH2, D)), W_B, W_C)
    beta = row[0, 0] @ W_B
    assert np.array_equal(f.x[0, K], beta * (2.0 - 2.0 ** (1 - K)))
    assert np.array_equal(f.x[0, K], beta * 1.9921875)


def check_saturated_gates(orc):
    """Gate -> 0 keeps only the newest input; gate -> 1 sums every input.

    A constant feature h[:, :, 0] = 1 with W_A[0, :] = -60 and the rest of W_A
    zero gives a = -60 exactly, sigma(-60) ~ 8.8e-27, so x_K = b_{K-1} to
    float64 precision.  W_A[0, :] = +60 gives sigma(60) = 1 in float64, so
    x_K = sum_t b_t.
    """
    rng = np.random.default_rng(303)
    B, K, SH2, D = 4, 6, 7, 3
    H = rng.standard_normal((B, K, SH2))
    H[:, :, 0] = 1.0
    h_s2 = rng.standard_normal((B, SH2))
    W_B = rng.uniform(-0.5, 0.5, (SH2, D))
    W_C = rng.uniform(-0.5, 0.5, (SH2, D))
    bt = np.einsum("bkj,js->bks", H, W_B)  # reference b_t (independent of orc)
    for sign, expect in ((-1.0, bt[:, K - 1]), (1.0, bt.sum(axis=1))):
        W_A = np.zeros((SH2, D))
        W_A[0, :] = 60.0 * sign
        f = orc.forward(H, h_s2, W_A, W_B, W_C)
        np.testing.assert_allclose(f.x[:, K], expect, rtol=1e-12, atol=1e-12)


def check_gate_matches_expit(orc):
    """K = 2 with generic logits: x_2 = expit(a_1) * b_0 + b_1.

    The projections are brute-force sums (math.fsum over explicit products)
    and the gate is scipy's expit, so neither reuses the oracle's routines.
    Also checks that extreme logits give gates in [0, 1] without overflow.
    """
    rng = np.random.default_rng(404)
    B, K, SH2, D = 3, 2, 9, 4
    H, h_s2, W_A, W_B, W_C, _ = _real_inputs(rng, B, K, SH2, D, wa_scale=1.5)
    f = orc.forward(H, h_s2, W_A, W_B, W_C)
    for b in range(B):
        for s in range(D):
            a1 = math.fsum(H[b, 1, j] * W_A[j, s] for j in range(SH2))
            b0 = math.fsum(H[b, 0, j] * W_B[j, s] for j in range(SH2))
            b1 = math.fsum(H[b, 1, j] * W_B[j, s] for j in range(SH2))
            c = math.fsum(h_s2[b, j] * W_C[j, s] for j in range(SH2))
            x2 = expit(a1) * b0 + b1
            assert abs(f.x[b, 2, s] - x2) <= 1e-13 * (1 + abs(x2)), (b, s)
            assert abs(f.context[b, s] - c * x2) <= 1e-13 * (1 + abs(c * x2)), (b, s)
    with np.errstate(over="raise", invalid="raise"):
        g = orc.logistic(np.array([-800.0, -60.0, 0.0, 60.0, 800.0]))
    assert np.all((g >= 0) & (g <= 1)) and np.all(np.isfinite(g))
    np.testing.assert_allclose(g, expit(np.array([-800.0, -60.0, 0.0, 60.0, 800.0])), rtol=1e-15)


# --------------------------------------------------------------- backward pins
def _fd_grad(fun, X, h):
    G = np.empty_like(X)
    for idx in np.ndindex(X.shape):
        old = X[idx]
        X[idx] = old + h
        lp = fun()
        X[idx] = old - h
        lm = fun()
        X[idx] = old
        G[idx] = (lp - lm) / (2 * h)
    return G


def check_weight_grads_finite_difference(orc):
    """Central differences of L = sum(d_context * context) for every W entry.

    Shapes (B, K, SH2, D) = (3, 4, 5, 2), (2, 1, 3, 2), (2, 7, 4, 3); h = 1e-6.
    Only the oracle's forward enters the differences, so this pins the whole
    backward against it.
    """
    rng = np.random.default_rng(505)
    for B, K, SH2, D in ((3, 4, 5, 2), (2, 1, 3, 2), (2, 7, 4, 3)):
        H, h_s2, W_A, W_B, W_C, d_ctx = _real_inputs(rng, B, K, SH2, D, wa_scale=1.0)
        f = orc.forward(H, h_s2, W_A, W_B, W_C)
        g = orc.backward(f, H, h_s2, d_ctx)

        def L():
            ff = orc.forward(H, h_s2, W_A, W_B, W_C)
            return float(np.sum(d_ctx * ff.context))

        for W, an in ((W_A, g.dW_A), (W_B, g.dW_B), (W_C, g.dW_C)):
            fd = _fd_grad(L, W, 1e-6)
            scale = max(1.0, float(np.max(np.abs(an))))
            err = float(np.max(np.abs(fd - an)))
            assert err <= 2e-8 * scale, ((B, K, SH2, D), err, scale)


def check_intermediate_grads_finite_difference(orc):
    """Central differences of L with respect to a, b and c themselves.

    Pins d_a, d_b and d_c (the reverse scan alone) at (B, K, D) = (2, 5, 3).
    """
    rng = np.random.default_rng(606)
    B, K, SH2, D = 2, 5, 4, 3
    H, h_s2, W_A, W_B, W_C, d_ctx = _real_inputs(rng, B, K, SH2, D, wa_scale=1.0)
    f = orc.forward(H, h_s2, W_A, W_B, W_C)
    g = orc.backward(f, H, h_s2, d_ctx)
    a = f.a.copy()
    bb = f.bb.copy()
    c = f.c.copy()

    def L():
        return float(np.sum(d_ctx * orc.context_from_projections(a, bb, c)))

    for X, an in ((a, g.d_a), (bb, g.d_b), (c, g.d_c)):
        fd = _fd_grad(L, X, 1e-6)
        err = float(np.max(np.abs(fd - an)))
        assert err <= 2e-8 * max(1.0, float(np.max(np.abs(an)))), err


def check_reverse_scan_products(orc):
    """Closed form of the reverse scan, by products instead of recursion.

    d_b[t] = d_context * c * prod_{u>t} g_u, d_a[t] = d_b[t] * x_t * g_t (1 - g_t),
    d_c = d_context * x_K.  The gates come from scipy's expit applied to the
    oracle's logits.
    """
    rng = np.random.default_rng(707)
    B, K, SH2, D = 3, 6, 5, 4
    H, h_s2, W_A, W_B, W_C, d_ctx = _real_inputs(rng, B, K, SH2, D, wa_scale=1.0)
    f = orc.forward(H, h_s2, W_A, W_B, W_C)
    g = orc.backward(f, H, h_s2, d_ctx)
    gate = expit(f.a)
    for t in range(K):
        suffix = np.prod(gate[:, t + 1:], axis=1) if t + 1 < K else np.ones((B, D))
        db = d_ctx * f.c * suffix
        np.testing.assert_allclose(g.d_b[:, t], db, rtol=1e-13, atol=1e-15)
        da = db * f.x[:, t] * gate[:, t] * (1 - gate[:, t])
        np.testing.assert_allclose(g.d_a[:, t], da, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(g.d_c, d_ctx * f.x[:, K], rtol=1e-14, atol=0)


def check_k1_no_gate_gradient(orc):
    """K = 1: x_0 = 0 makes d_a identically zero, so dW_A is exactly zero."""
    rng = np.random.default_rng(808)
    H, h_s2, W_A, W_B, W_C, d_ctx = _real_inputs(rng, 4, 1, 6, 3)
    f = orc.forward(H, h_s2, W_A, W_B, W_C)
    g = orc.backward(f, H, h_s2, d_ctx)
    assert np.all(g.d_a == 0.0) and np.all(g.dW_A == 0.0)
    assert np.any(g.dW_B != 0.0) and np.any(g.dW_C != 0.0)


def check_invariants(orc):
    """Batch additivity, sample permutation, linearity in d_context, homogeneity.

    * dW over all samples = dW(first part) + dW(rest), for any split.
    * Permuting samples permutes context rows and leaves dW unchanged.
    * The backward is linear in d_context.
    * context(l * W_B) = l * context and context(l * W_C) = l * context.
    """
    rng = np.random.default_rng(909)
    B, K, SH2, D = 7, 5, 6, 4
    H, h_s2, W_A, W_B, W_C, d_ctx = _real_inputs(rng, B, K, SH2, D, wa_scale=1.0)

    def run(Hh, hs, dc):
        f = orc.forward(Hh, hs, W_A, W_B, W_C)
        return f, orc.backward(f, Hh, hs, dc)

    f, g = run(H, h_s2, d_ctx)
    for cut in (1, 3, 6):
        _, g1 = run(H[:cut], h_s2[:cut], d_ctx[:cut])
        _, g2 = run(H[cut:], h_s2[cut:], d_ctx[cut:])
        for name in ("dW_A", "dW_B", "dW_C"):
            np.testing.assert_allclose(getattr(g1, name) + getattr(g2, name), getattr(g, name),
                                       rtol=1e-12, atol=1e-12)
    perm = rng.permutation(B)
    fp, gp = run(H[perm], h_s2[perm], d_ctx[perm])
    np.testing.assert_allclose(fp.context, f.context[perm], rtol=1e-14, atol=0)
    for name in ("dW_A", "dW_B", "dW_C"):
        np.testing.assert_allclose(getattr(gp, name), getattr(g, name), rtol=1e-12, atol=1e-12)
    d2 = rng.standard_normal((B, D))
    _, gb = run(H, h_s2, d2)
    _, gl = run(H, h_s2, 2.5 * d_ctx - 0.75 * d2)
    for name in ("dW_A", "dW_B", "dW_C", "d_a", "d_b", "d_c"):
        np.testing.assert_allclose(getattr(gl, name), 2.5 * getattr(g, name) - 0.75 * getattr(gb, name),
                                   rtol=1e-11, atol=1e-12)
    fb = orc.forward(H, h_s2, W_A, 3.0 * W_B, W_C)
    fc = orc.forward(H, h_s2, W_A, W_B, -2.0 * W_C)
    np.testing.assert_allclose(fb.context, 3.0 * f.context, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fc.context, -2.0 * f.context, rtol=1e-12, atol=1e-13)


def check_input_grads_finite_difference(orc):
    """Central differences of L with respect to every entry of h_history and h_s2.

    Shapes (B, K, SH2, D) = (2, 3, 4, 2) and (1, 1, 3, 3); h = 1e-6.  Only
    the oracle's forward enters the differences.
    """
    rng = np.random.default_rng(1010)
    for B, K, SH2, D in ((2, 3, 4, 2), (1, 1, 3, 3)):
        H, h_s2, W_A, W_B, W_C, d_ctx = _real_inputs(rng, B, K, SH2, D, wa_scale=1.0)
        f = orc.forward(H, h_s2, W_A, W_B, W_C)
        g = orc.input_grads(orc.backward(f, H, h_s2, d_ctx), W_A, W_B, W_C)

        def L():
            ff = orc.forward(H, h_s2, W_A, W_B, W_C)
            return float(np.sum(d_ctx * ff.context))

        for X, an in ((H, g.d_h_history), (h_s2, g.d_h_s2)):
            fd = _fd_grad(L, X, 1e-6)
            err = float(np.max(np.abs(fd - an)))
            assert err <= 2e-8 * max(1.0, float(np.max(np.abs(an)))), ((B, K, SH2, D), err)


# ------------------------------------------- stability multiplier and blend
def check_stability_geometric(orc):
    """W_A = 0 gives sigma = 1/2; with multiplier m the gate is m/2.

    Rows equal across t give b_t = beta (an integer), so with m = 1/2:
    x_K = beta * sum_{i<K} 4^-i exactly, and context = c * x_K exactly.  With
    m = 0 only the newest input survives: x_K = b_{K-1}.  (A multiplier that
    scaled the input instead of the gate would give beta * sum 2^-i * 1/2.)
    """
    rng = np.random.default_rng(1111)
    B, K, SH2, D = 3, 6, 5, 2
    H, h_s2, W_A, W_B, W_C = _int_inputs(rng, B, K, SH2, D)
    W_A[:] = 0.0
    Heq = np.repeat(H[:, :1], K, axis=1)
    f = orc.forward(Heq, h_s2, W_A, W_B, W_C, stability=0.5)
    geo = sum(Fraction(1, 4 ** i) for i in range(K))
    for b in range(B):
        for s in range(D):
            beta = _dot_int(Heq[b, 0], W_B[:, s])
            c = _dot_int(h_s2[b], W_C[:, s])
            assert f.x[b, K, s] == float(beta * geo), (b, s)
            assert f.context[b, s] == float(c * beta * geo), (b, s)
    f0 = orc.forward(H, h_s2, W_A, W_B, W_C, stability=0.0)
    for b in range(B):
        for s in range(D):
            assert f0.x[b, K, s] == _dot_int(H[b, K - 1], W_B[:, s]), (b, s)


def check_stability_backward_products(orc):
    """Reverse scan with multiplier m, by products: d_b[t] = d_context c prod_{u>t} m g_u,
    d_a[t] = d_b[t] x_t m g_t (1 - g_t), with g = scipy expit of the oracle's logits."""
    rng = np.random.default_rng(1212)
    B, K, SH2, D = 3, 5, 4, 3
    H, h_s2, W_A, W_B, W_C, d_ctx = _real_inputs(rng, B, K, SH2, D, wa_scale=1.0)
    m = 0.7
    f = orc.forward(H, h_s2, W_A, W_B, W_C, stability=m)
    g = orc.backward(f, H, h_s2, d_ctx)
    gate = expit(f.a)
    # the forward itself, by the same closed form: x_{t+1} = m g_t x_t + b_t
    x = np.zeros((B, D))
    for t in range(K):
        x = m * gate[:, t] * x + f.bb[:, t]
    np.testing.assert_allclose(f.x[:, K], x, rtol=1e-13, atol=1e-14)
    for t in range(K):
        suffix = np.prod(m * gate[:, t + 1:], axis=1) if t + 1 < K else np.ones((B, D))
        db = d_ctx * f.c * suffix
        np.testing.assert_allclose(g.d_b[:, t], db, rtol=1e-13, atol=1e-15)
        da = db * f.x[:, t] * m * gate[:, t] * (1 - gate[:, t])
        np.testing.assert_allclose(g.d_a[:, t], da, rtol=1e-12, atol=1e-15)


def check_blend_closed_form(orc):
    """K = 1, integer inputs, D = 4: h_enriched = h_s2 + w * (sum_s c x_1) / 4, exactly.

    x_1 = b_0, every product and the division by a power of two are exact in
    float64.  Also w absent means w = 1.
    """
    rng = np.random.default_rng(1313)
    B, K, SH2, D = 3, 1, 5, 4
    H, h_s2, W_A, W_B, W_C = _int_inputs(rng, B, K, SH2, D)
    w = rng.integers(-3, 4, SH2).astype(np.float64)
    f = orc.forward(H, h_s2, W_A, W_B, W_C)
    he = orc.blend(f.context, h_s2, w)
    he1 = orc.blend(f.context, h_s2)
    for b in range(B):
        tot = sum(_dot_int(h_s2[b], W_C[:, s]) * _dot_int(H[b, 0], W_B[:, s]) for s in range(D))
        for j in range(SH2):
            assert he[b, j] == float(Fraction(int(h_s2[b, j])) + int(w[j]) * Fraction(tot, D)), (b, j)
            assert he1[b, j] == float(Fraction(int(h_s2[b, j])) + Fraction(tot, D)), (b, j)


def check_blend_finite_difference(orc):
    """Central differences of L = sum(d_h_enriched * h_enriched) through the blend.

    With a stability multiplier (0.8, 1.3) and temporal weights (random, or
    absent): every entry of W_A, W_B, W_C, the temporal weights and h_s2 (whose
    gradient is the residual plus the W_C path).  h = 1e-6.
    """
    rng = np.random.default_rng(1414)
    for (B, K, SH2, D), m, with_w in (((3, 4, 5, 2), 0.8, True), ((2, 7, 3, 4), 1.3, False)):
        H, h_s2, W_A, W_B, W_C, _ = _real_inputs(rng, B, K, SH2, D, wa_scale=1.0)
        w = rng.uniform(0.5, 1.5, SH2) if with_w else None
        dhe = rng.standard_normal((B, SH2))
        inp = dict(h_history=H, h_s2=h_s2, W_A=W_A, W_B=W_B, W_C=W_C, d_h_enriched=dhe)
        _, _, bb, b = orc.fwd_bwd_blend(inp, m, w)
        d_hs2 = bb.d_h_s2_residual + orc.input_grads(b, W_A, W_B, W_C).d_h_s2

        def L():
            return orc.loss_blend(H, h_s2, W_A, W_B, W_C, dhe, m, w)

        checks = [(W_A, b.dW_A), (W_B, b.dW_B), (W_C, b.dW_C), (h_s2, d_hs2)]
        if w is not None:
            checks.append((w, bb.d_temporal_weight))
        for X, an in checks:
            fd = _fd_grad(L, X, 1e-6)
            err = float(np.max(np.abs(fd - an)))
            assert err <= 2e-8 * max(1.0, float(np.max(np.abs(an)))), ((B, K, SH2, D), m, err)


ALL_PINS = [
    check_k1_closed_form,
    check_half_gate_geometric,
    check_saturated_gates,
    check_gate_matches_expit,
    check_weight_grads_finite_difference,
    check_intermediate_grads_finite_difference,
    check_reverse_scan_products,
    check_k1_no_gate_gradient,
    check_invariants,
    check_input_grads_finite_difference,
    check_stability_geometric,
    check_stability_backward_products,
    check_blend_closed_form,
    check_blend_finite_difference,
]
