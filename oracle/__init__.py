"""fp64 CPU oracle (test infrastructure only; see rope_oracle's module docstring)."""
from .rope_oracle import *  # noqa: F401,F403
