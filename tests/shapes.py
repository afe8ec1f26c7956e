"""Shape lists of the GPU parity tests (B, K, SH2, STATE_D).

Kept apart from the GPU test modules so that a CPU test
(tests/test_launch_forms.py) can check, through the library's own launch
plan, that these lists reach every forward launch form.  The lists hold
dimensions only; the inputs come from tests/inputs.py.
"""
from __future__ import annotations

from tests.inputs import WORKLOADS

# One sample, ragged batches (B % 16 != 0), K = 1, K across the 8-step
# projection rounds (9, 17, 64, 80, 100), every SH2 multiple of 64 from 64 to
# 512, all three state widths, and partial slices in the backward.
EDGE_SHAPES = [
    (1, 1, 64, 16),
    (1, 8, 256, 16),
    (17, 3, 128, 16),
    (33, 9, 256, 16),
    (5, 17, 192, 32),
    (40, 8, 320, 64),
    (16, 8, 512, 64),
    (100, 2, 448, 16),
    (64, 64, 256, 16),
    (3, 8, 384, 32),
    (250, 5, 64, 64),
    (129, 1, 512, 32),
    (300, 12, 256, 16),
    (20, 80, 64, 16),     # ten 8-step rounds: two beyond those held in registers
    (5, 100, 128, 32),
    (7, 20, 128, 64),     # four state groups over three rounds
]

# Long histories with few samples: the forward cuts the history into chunks
# that run in parallel (summary pass, carry across chunks, replay pass).
LONG_FEW_SHAPES = [
    (64, 1024, 256, 16),
    (8, 2048, 128, 32),
    (3, 300, 64, 64),
    (17, 160, 192, 16),
    (5, 8192, 64, 16),    # one sample block: 512 history chunks, the carry's 32 segments
    (20, 96, 384, 16),    # a wide trunk in chunks: one-block summary pass, two-block replay
    (32, 2024, 256, 16),  # 63 chunks of 32 steps, the remainder merged into a 40-step last chunk
    (32, 2040, 256, 16),  # 64 chunks, the last one 24 steps
]

# The launch forms of wide trunks (SH2 >= 320, where a work-group may hold two
# 16-sample blocks), each in fp32 and bf16.
FORM_SHAPES = [
    # two-block full pass (enough pairs of blocks to fill the GPU); 129
    # blocks, so the second block of the last pair lies past the batch
    (2050, 3, 320, 64),
    (2050, 2, 384, 64),
    (2050, 2, 448, 64),
    (2050, 2, 512, 64),
    (8200, 2, 320, 16),   # one state group: 257 pairs
    # chunked history, few blocks: one-block summary pass, carry, two-block replay
    (20, 96, 320, 16),
    (20, 96, 448, 16),
    (5, 64, 512, 16),
    # chunked history, enough pairs for the two-block summary pass; 63
    # blocks (odd), ragged last block
    (1000, 48, 320, 64),
    (1000, 48, 384, 64),
    (1000, 48, 448, 64),
    (1000, 48, 512, 64),
]

# Shapes whose history is long enough to be chunked run with long-memory
# gates (+2 logit shift), so that the carry across chunks matters.
def gate_bias(K: int) -> float:
    return 2.0 if K >= 32 else 0.0


# bf16 trunk inputs: the chunked shapes of tests/test_bf16_gpu.py
BF16_CHUNKED_SHAPES = [(64, 1024, 256, 16), (3, 300, 64, 64), (17, 160, 192, 16), (20, 96, 384, 16)]

# Workloads run end to end against the oracle, per trunk precision.
FP32_WORKLOADS = ["tiny", "mid", "pages_shape", "long_history", "wide_state", "long_few"]
BF16_WORKLOADS = ["tiny", "mid", "pages_shape", "long_history", "wide_state"]


def _wl(names):
    return [(WORKLOADS[n].B, WORKLOADS[n].K, WORKLOADS[n].SH2, WORKLOADS[n].D) for n in names]


# Every shape whose forward the parity tests compare with the oracle.
FP32_FWD_SHAPES = EDGE_SHAPES + LONG_FEW_SHAPES + FORM_SHAPES + _wl(FP32_WORKLOADS)
BF16_FWD_SHAPES = EDGE_SHAPES + BF16_CHUNKED_SHAPES + FORM_SHAPES + _wl(BF16_WORKLOADS)
