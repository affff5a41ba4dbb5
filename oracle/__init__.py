"""CPU oracle of the MoE layer (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
