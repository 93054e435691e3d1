"""CPU oracle of the one-GPU MoE layer (test infrastructure only)."""
from .oracle import *  # noqa: F401,F403
