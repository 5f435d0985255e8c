"""CPU oracle (test infrastructure only; see w4_oracle.py's header)."""
from .w4_oracle import *  # noqa: F401,F403
from . import w4_oracle  # noqa: F401
