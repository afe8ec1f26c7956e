"""Seeded synthetic inputs for the Mamba2 temporal scan.

This module only draws random numbers; it holds none of the scan's arithmetic.
The oracle and the HIP path both consume the host arrays it returns.

The workloads follow the shapes of the foxhunt pages ("Custom Kernel
Optimization Implementation Plan", header dimensions; design spec, nsys
breakdown at batch 8192): trunk width SH2, state width STATE_D, history
length K and batch B.  The pages train on a futures dataset that is not
available here; i.i.d. draws of the same shapes stand in for it.

Draw order (numpy PCG64, seed = the config's index unless given):
  1. h_history ~ N(0, 1), shape (B, K, SH2), float32
  2. h_s2      ~ N(0, 1), shape (B, SH2), float32
  3. W_A, W_B, W_C ~ U(-r, r), shape (SH2, STATE_D), r = 1/sqrt(SH2), float32
  4. d_context ~ N(0, 1), shape (B, STATE_D), float32
The long-history workload then sets the constant feature h_history[:, :, 0] = 1
and adds 2 to W_A[0, :], so every gate logit is shifted by +2 and the mean gate
is near sigmoid(2) ~ 0.88 (long memory).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    SH2: int
    D: int
    seed: int
    gate_bias: float = 0.0  # added to W_A[0, :] with h_history[:, :, 0] = 1


# The workloads: a tiny case the oracle finishes instantly, a mid case, the
# pages' own shape (B=8192, K=8, SH2=256, STATE_D=16), a long history with
# long-memory gates, a wide state, and a long history with few samples.
WORKLOADS = {
    "tiny": Workload("tiny", 64, 8, 256, 16, seed=0),
    "mid": Workload("mid", 1024, 8, 256, 16, seed=1),
    "pages_shape": Workload("pages_shape", 8192, 8, 256, 16, seed=2),
    "long_history": Workload("long_history", 8192, 64, 256, 16, seed=3, gate_bias=2.0),
    "wide_state": Workload("wide_state", 32768, 8, 512, 64, seed=4),
    # a long history with few samples (the forward runs its chunks in parallel)
    "long_few": Workload("long_few", 128, 2048, 256, 16, seed=5, gate_bias=2.0),
}


def make_inputs(B: int, K: int, SH2: int, D: int, seed: int, gate_bias: float = 0.0):
    """Return a dict of float32 host arrays in the fixed draw order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    h_history = rng.standard_normal((B, K, SH2), dtype=np.float32)
    h_s2 = rng.standard_normal((B, SH2), dtype=np.float32)
    r = 1.0 / np.sqrt(SH2)
    W_A = rng.uniform(-r, r, (SH2, D)).astype(np.float32)
    W_B = rng.uniform(-r, r, (SH2, D)).astype(np.float32)
    W_C = rng.uniform(-r, r, (SH2, D)).astype(np.float32)
    d_context = rng.standard_normal((B, D), dtype=np.float32)
    if gate_bias != 0.0:
        h_history[:, :, 0] = 1.0
        W_A[0, :] += np.float32(gate_bias)
    return {
        "h_history": h_history,
        "h_s2": h_s2,
        "W_A": W_A,
        "W_B": W_B,
        "W_C": W_C,
        "d_context": d_context,
    }


def workload_inputs(name: str):
    w = WORKLOADS[name]
    return make_inputs(w.B, w.K, w.SH2, w.D, w.seed, w.gate_bias)


def blend_extras(B: int, SH2: int, seed: int):
    """Inputs of the h_enriched blend, drawn from their own stream (seed + 1000).

    Draw order: d_h_enriched ~ N(0, 1), shape (B, SH2); temporal_weight ~
    U(0.5, 1.5), shape (SH2,); both float32.
    """
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    return {
        "d_h_enriched": rng.standard_normal((B, SH2), dtype=np.float32),
        "temporal_weight": rng.uniform(0.5, 1.5, SH2).astype(np.float32),
    }


def bf16_round(x):
    """Round float32 values to bfloat16 (nearest, ties to even).

    Returns (bits, values): the 16-bit patterns (uint16) the reduced-precision
    entry points take, and the same values widened back to float32 for the
    oracle and the fp32 entry points.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    values = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits, values
