"""fp64 CPU oracles (test infrastructure only; see each module's header): the MoE layer, GQA
decode attention over a block-paged KV cache, and the gated delta-rule recurrence."""
from . import attn_oracle, delta_oracle, moe_oracle  # noqa: F401
