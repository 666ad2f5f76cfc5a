"""CPU oracle (test infrastructure only; see tq_oracle.py)."""
from .tq_oracle import *  # noqa: F401,F403
