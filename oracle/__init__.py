"""fp64 CPU oracle for FAVOR+ (test infrastructure only; see favor_oracle.py)."""
from .favor_oracle import *  # noqa: F401,F403
from .favor_oracle import __all__  # noqa: F401
