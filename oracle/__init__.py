"""CPU oracle of the MoE layer (test infrastructure; see moe_oracle's header)."""
from . import moe_oracle  # noqa: F401
