"""CPU oracle (test infrastructure only; see mamba2_oracle's header)."""
from . import mamba2_oracle  # noqa: F401
