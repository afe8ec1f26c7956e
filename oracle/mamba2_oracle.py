"""CPU oracle for the Mamba2 temporal scan, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The HIP library never
calls it and shares no code with it.

Everything is plain numpy in float64: inputs are widened from float32, every
step is the textbook definition, written in the order the pages give it.  A
library matrix product serves as the projection step; nothing is blocked,
fused or reordered beyond that.

Sources (foxhunt pages):
  * "Custom Kernel Optimization Implementation Plan", Task 1 (Mamba2 forward:
    cuBLAS projections + lightweight scan) and Task 2 (Mamba2 backward: reverse
    scan + weight-gradient GEMMs).
  * "Custom Kernel Optimization -- cuBLAS Projections + Batch-Parallel Scans",
    Design section 1 (Mamba2 scan: forward steps 1-2, backward steps 1-3).

Notation: H = h_history[B, K, SH2] (row b*K+t of the flattened [B*K, SH2]
matrix is sample b at history step t; t = K-1 is the newest), h_s2[B, SH2],
W_A, W_B, W_C[SH2, D] (element (j, s) is row j, column s), D = STATE_D.

Readings taken where the pages are silent or disagree (each also listed in the
design notes):
  * context is per state: context[b, s] = c[b, s] * x_K[b, s] (design spec,
    forward step 2); the plan's sum over s into h_enriched is a later step.
  * W_C projects h_s2 in the forward (both pages), so upstream d_context[B, D]
    is given and dW_C = h_s2^T d_c with d_c = d_context * x_K.
  * The reverse scan starts from dx_K = d_context * c (chain rule; the plan's
    comment states it, its code line drops the factor c).
  * x_0 = 0, no biases.  The stability multiplier (the plan's optional
    isv_signals[11] factor) defaults to 1, the pages' main path; when given
    it scales the gate in the recurrence and both derivative factors (plan
    Task 1 step 3, Task 2 step 2).
  * Weight gradients overwrite; they are not accumulated into.
  * The h_enriched blend (plan Task 1 step 3) is the step after the path:
    h_enriched[b, j] = h_s2[b, j] + w_j * (sum_s context[b, s]) / D with
    w_j = temporal_weight[j] (1 when absent).  Its backward follows the chain
    rule: d_context[b, s] = sum_j d_h_enriched[b, j] w_j / D for every s,
    d_temporal_weight[j] = sum_b d_h_enriched[b, j] (sum_s context[b, s]) / D,
    and d_h_enriched passes unchanged to h_s2 through the residual.  (The
    plan's backward listing instead contracts d_h_enriched with W_C; that
    treats W_C as an output projection, which its forward does not.)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def project(rows, W) -> np.ndarray:
    """Projection rows @ W in float64.

    Plan, Task 1 step 2 / design spec forward step 1: A_vals = h_history @ W_A,
    B_vals = h_history @ W_B over the flattened [B*K, SH2] history, and
    C_vals = h_s2 @ W_C.
    """
    return _f64(rows) @ _f64(W)


def logistic(a) -> np.ndarray:
    """Gate sigma(a) = 1 / (1 + exp(-a)) (plan Task 1 step 3; design spec step 2).

    For a < 0 the equal form exp(a) / (1 + exp(a)) is used so that no
    intermediate overflows; the value is the same function.
    """
    a = _f64(a)
    out = np.empty_like(a)
    pos = a >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-a[pos]))
    e = np.exp(a[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def scan_forward(a, bb, m=1.0):
    """Gated recurrence over the K history steps for every (sample, state).

    x_0 = 0 and x_{t+1} = (m * sigma(a_t)) * x_t + b_t for t = 0 .. K-1 in
    storage order (plan Task 1 step 3; design spec forward step 2), with m
    the stability multiplier (1 on the pages' main path).

    Returns (g[B, K, D], x[B, K+1, D]) with g = sigma(a) (without m), x[:, t]
    the state *before* step t is applied and x[:, K] the final state.
    """
    a = _f64(a)
    bb = _f64(bb)
    m = float(m)
    B, K, D = a.shape
    g = logistic(a)
    x = np.zeros((B, K + 1, D))
    for t in range(K):
        x[:, t + 1] = (m * g[:, t]) * x[:, t] + bb[:, t]
    return g, x


@dataclass
class Forward:
    a: np.ndarray        # [B, K, D] gate logits  H @ W_A
    bb: np.ndarray       # [B, K, D] inputs       H @ W_B
    c: np.ndarray        # [B, D]    readout      h_s2 @ W_C
    g: np.ndarray        # [B, K, D] sigma(a)
    x: np.ndarray        # [B, K+1, D] states, x[:, 0] = 0
    context: np.ndarray  # [B, D]    c * x_K
    m: float = 1.0       # stability multiplier of the gate


def forward(h_history, h_s2, W_A, W_B, W_C, stability=1.0) -> Forward:
    """Forward pass: three projections, the scan, then context = c * x_K."""
    H = _f64(h_history)
    B, K, SH2 = H.shape
    rows = H.reshape(B * K, SH2)
    a = project(rows, W_A).reshape(B, K, -1)
    bb = project(rows, W_B).reshape(B, K, -1)
    c = project(h_s2, W_C)
    g, x = scan_forward(a, bb, stability)
    context = c * x[:, K]
    return Forward(a=a, bb=bb, c=c, g=g, x=x, context=context, m=float(stability))


def context_from_projections(a, bb, c, m=1.0) -> np.ndarray:
    """context = c * x_K from given projections (used to differentiate numerically)."""
    _, x = scan_forward(a, bb, m)
    return _f64(c) * x[:, -1]


def scan_backward(g, x, c, d_context, m=1.0):
    """Reverse scan (plan Task 2 step 2; design spec backward step 2).

    L = sum_{b,s} d_context[b, s] * context[b, s] defines every gradient.
      dx_K = d_context * c          d_c = d_context * x_K
      for t = K-1 down to 0:
        d_b[t] = dx_t
        d_a[t] = dx_t * x_t * sigma'(a_t) * m,  sigma' = g * (1 - g)
        dx_{t}  <- dx_t * g_t * m   (gradient w.r.t. the state before step t)
    with m the stability multiplier (1 on the main path).  The last dx (w.r.t.
    x_0 = 0, a constant) is discarded.
    """
    g = _f64(g)
    x = _f64(x)
    d_context = _f64(d_context)
    m = float(m)
    B, K, D = g.shape
    dx = d_context * _f64(c)
    d_c = d_context * x[:, K]
    d_a = np.empty((B, K, D))
    d_b = np.empty((B, K, D))
    for t in range(K - 1, -1, -1):
        gt = g[:, t]
        d_b[:, t] = dx
        d_a[:, t] = dx * x[:, t] * gt * (1.0 - gt) * m
        dx = dx * gt * m
    return d_a, d_b, d_c


@dataclass
class Backward:
    d_a: np.ndarray   # [B, K, D]
    d_b: np.ndarray   # [B, K, D]
    d_c: np.ndarray   # [B, D]
    dW_A: np.ndarray  # [SH2, D]
    dW_B: np.ndarray  # [SH2, D]
    dW_C: np.ndarray  # [SH2, D]


def backward(fwd: Forward, h_history, h_s2, d_context) -> Backward:
    """Backward pass: reverse scan, then the three weight-gradient products.

    dW_A = H^T d_a and dW_B = H^T d_b over the B*K history rows, and
    dW_C = h_s2^T d_c over the B samples (plan Task 2 step 3; design spec
    backward step 3).
    """
    H = _f64(h_history)
    B, K, SH2 = H.shape
    d_a, d_b, d_c = scan_backward(fwd.g, fwd.x, fwd.c, d_context, fwd.m)
    rows = H.reshape(B * K, SH2)
    D = d_c.shape[1]
    dW_A = rows.T @ d_a.reshape(B * K, D)
    dW_B = rows.T @ d_b.reshape(B * K, D)
    dW_C = _f64(h_s2).T @ d_c
    return Backward(d_a=d_a, d_b=d_b, d_c=d_c, dW_A=dW_A, dW_B=dW_B, dW_C=dW_C)


@dataclass
class InputGrads:
    d_h_history: np.ndarray  # [B, K, SH2]
    d_h_s2: np.ndarray       # [B, SH2]


def input_grads(bwd: Backward, W_A, W_B, W_C) -> InputGrads:
    """Gradients of L with respect to the trunk inputs.

    The pages stop at the weight gradients (plan Task 2 ends with the
    weight-gradient GEMMs); training the trunk through the scan also needs
    dL/dh_history and dL/dh_s2.  By the chain rule through the three
    projections of plan Task 1 step 2:
      d_h_history[b, t, :] = d_a[b, t, :] @ W_A^T + d_b[b, t, :] @ W_B^T
      d_h_s2[b, :]         = d_c[b, :] @ W_C^T
    """
    B, K, D = bwd.d_a.shape
    d_a = bwd.d_a.reshape(B * K, D)
    d_b = bwd.d_b.reshape(B * K, D)
    dH = d_a @ _f64(W_A).T + d_b @ _f64(W_B).T
    dhs2 = bwd.d_c @ _f64(W_C).T
    return InputGrads(d_h_history=dH.reshape(B, K, -1), d_h_s2=dhs2)


def blend(context, h_s2, temporal_weight=None) -> np.ndarray:
    """h_enriched = h_s2 + w * (sum_s context) / D (plan Task 1 step 3, the residual blend).

    w = temporal_weight [SH2], or 1 for every feature when absent.
    """
    ctx = _f64(context)
    D = ctx.shape[1]
    ctx_sum = ctx.sum(axis=1)
    h = _f64(h_s2)
    w = np.ones(h.shape[1]) if temporal_weight is None else _f64(temporal_weight)
    return h + w[None, :] * ctx_sum[:, None] * (1.0 / D)


@dataclass
class BlendBackward:
    d_context: np.ndarray          # [B, D]: the same value for every state of a sample
    d_temporal_weight: np.ndarray  # [SH2]
    d_h_s2_residual: np.ndarray    # [B, SH2]: d_h_enriched itself


def blend_backward(d_h_enriched, context, temporal_weight=None) -> BlendBackward:
    """Chain rule through the blend (the reading stated in this module's header)."""
    dhe = _f64(d_h_enriched)
    ctx = _f64(context)
    B, D = ctx.shape
    w = np.ones(dhe.shape[1]) if temporal_weight is None else _f64(temporal_weight)
    d_sum = (dhe @ w) * (1.0 / D)                   # dL / d(sum_s context[b, s])
    d_context = np.repeat(d_sum[:, None], D, axis=1)
    d_w = dhe.T @ ctx.sum(axis=1) * (1.0 / D)
    return BlendBackward(d_context=d_context, d_temporal_weight=d_w, d_h_s2_residual=dhe.copy())


def fwd_bwd_blend(inputs: dict, stability=1.0, temporal_weight=None, d_h_enriched=None):
    """Forward with the stability multiplier and the blend, then the chain back to the weights.

    d_h_enriched defaults to inputs["d_h_enriched"].  Returns (fwd, h_enriched,
    blend_bwd, bwd).
    """
    f = forward(inputs["h_history"], inputs["h_s2"], inputs["W_A"], inputs["W_B"], inputs["W_C"], stability)
    he = blend(f.context, inputs["h_s2"], temporal_weight)
    dhe = inputs["d_h_enriched"] if d_h_enriched is None else d_h_enriched
    bb = blend_backward(dhe, f.context, temporal_weight)
    b = backward(f, inputs["h_history"], inputs["h_s2"], bb.d_context)
    return f, he, bb, b


def loss_blend(h_history, h_s2, W_A, W_B, W_C, d_h_enriched, stability=1.0, temporal_weight=None) -> float:
    """L = sum(d_h_enriched * h_enriched), whose gradients fwd_bwd_blend returns."""
    f = forward(h_history, h_s2, W_A, W_B, W_C, stability)
    return float(np.sum(_f64(d_h_enriched) * blend(f.context, h_s2, temporal_weight)))


def fwd_bwd(inputs: dict):
    """One forward + backward step on a dict from the seeded input generator."""
    f = forward(inputs["h_history"], inputs["h_s2"], inputs["W_A"], inputs["W_B"], inputs["W_C"])
    b = backward(f, inputs["h_history"], inputs["h_s2"], inputs["d_context"])
    return f, b

