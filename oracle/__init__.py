"""CPU oracle (test infrastructure only; see lizard_oracle's header)."""
from .lizard_oracle import *  # noqa: F401,F403
