"""CPU oracle for RRAttention (test infrastructure; see rra_oracle's header)."""
from .rra_oracle import *  # noqa: F401,F403
from .rra_oracle import __all__  # noqa: F401
