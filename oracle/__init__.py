"""CPU oracle of the MoE-layer forward pass (test infrastructure only)."""
from .moe_oracle import *  # noqa: F401,F403
