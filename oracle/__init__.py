"""CPU oracle of the MoE block (test infrastructure; see moe_oracle.py)."""
from .moe_oracle import *  # noqa: F401,F403
