"""CPU oracle for the CSA2 hot path (test infrastructure; see csa2_oracle)."""
from .csa2_oracle import *  # noqa: F401,F403
