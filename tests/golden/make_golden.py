"""Writes tests/golden/oracle_tiny.json from the oracle alone.

The foxhunt pages print no worked example for the Mamba2 scan, so this fixture
is not from the pages: it freezes the oracle's output on one tiny seeded input
(B=5, K=3, SH2=64, STATE_D=16, seed 7) so that a later change to the oracle's
arithmetic shows up as a test failure.  Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import mamba2_oracle as orc  # noqa: E402
from tests.inputs import make_inputs  # noqa: E402

SHAPE = dict(B=5, K=3, SH2=64, D=16, seed=7)


def main():
    inp = make_inputs(**SHAPE)
    f, b = orc.fwd_bwd(inp)
    out = {
        "source": "oracle/mamba2_oracle.py on tests/inputs.make_inputs(B=5, K=3, SH2=64, D=16, seed=7)",
        "shape": SHAPE,
        "context": f.context.tolist(),
        "dW_A": b.dW_A.tolist(),
        "dW_B": b.dW_B.tolist(),
        "dW_C": b.dW_C.tolist(),
    }
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as fh:
        json.dump(out, fh, indent=None, separators=(",", ":"))
        fh.write("\n")


if __name__ == "__main__":
    main()
