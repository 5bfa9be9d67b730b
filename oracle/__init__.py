"""CPU float64 oracle (test infrastructure only; see hm_oracle.py)."""
from .hm_oracle import *  # noqa: F401,F403
