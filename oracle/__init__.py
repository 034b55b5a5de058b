"""CPU float64 oracle (test infrastructure only; never imported by the product path)."""
from .flashforward import (  # noqa: F401
    GAMMA_BRACKET, GAMMA_CENTER_LR, ContractError, FFConfig, Rollout, anchor_positions,
    ar_depth, attention, attention_rows, chunk_positions, gamma, history_ids_after,
    is_legal_order, key_latents, n_anchors, n_chunks, planner_blocks, planner_key_blocks, schedule,
)
from .block_causal import (  # noqa: F401
    bc_backward, bc_complete_sources, bc_forward, bc_key_sources, bc_keys, bc_mask, source_rows,
)
