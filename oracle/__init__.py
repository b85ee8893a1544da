"""CPU oracle (test infrastructure only): plain float64 definitions of the
Q2_0 ternary linear, its low-rank branch and the 4-bit nibble variant."""
from .q2_oracle import *  # noqa: F401,F403
