"""fp64 CPU oracles (test infrastructure only; see each module's header): the MoE layer, GQA
decode attention over a block-paged KV cache, the gated delta-rule recurrence, and the greedy
decode step (LM head, argmax, embedding of the chosen token)."""
from . import attn_oracle, delta_oracle, head_oracle, moe_oracle  # noqa: F401
