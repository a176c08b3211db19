"""fp64 CPU oracle (test infrastructure only; see ttr_oracle)."""
from .ttr_oracle import *  # noqa: F401,F403
