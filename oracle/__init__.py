"""Float64 CPU oracle (test infrastructure only; see ttt_oracle.py)."""
from . import ttt_oracle  # noqa: F401
