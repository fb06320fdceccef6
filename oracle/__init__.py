"""Float64 CPU oracles (test infrastructure only): ``ttt_oracle.cpp`` (plain
C++, bound by ``cpp``) and ``ttt_oracle`` (numpy)."""
from . import ttt_oracle  # noqa: F401
