"""fp64 CPU oracle for the MoE layer (test infrastructure only; see moe_oracle's header)."""
from . import moe_oracle  # noqa: F401
