"""CPU oracle (test infrastructure only; see sffn_oracle.py)."""
from .sffn_oracle import *  # noqa: F401,F403
