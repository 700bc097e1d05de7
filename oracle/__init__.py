"""fp64 CPU oracle (test infrastructure only; see fsa_oracle's header)."""
from .fsa_oracle import *  # noqa: F401,F403
from .fsa_oracle import BETA  # noqa: F401
