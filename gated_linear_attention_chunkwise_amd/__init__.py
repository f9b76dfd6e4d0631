"""MI355X (gfx950) hybrid attention layer of Lizard: GLA with log-space
per-key-dimension gates plus an anchor window with meta-memory sinks.

The compute path is the HIP library liblizard_attn.so (built in-tree by
``gated_linear_attention_chunkwise_amd.build``); this package only binds it.
"""
from ._lib import (  # noqa: F401
    LizardError, Shape, SYMBOLS, lizard_attn_bwd, lizard_attn_decode_step, lizard_attn_fwd,
    lizard_attn_fwd_continue, load, make_shape, workspace_bytes, decode_workspace, continue_workspace,
    fwd, bwd, decode_step, fwd_continue, OP_FWD, OP_BWD, OP_DECODE, OP_FWD_CONTINUE, GATE_PER_DIM,
    GATE_SCALAR, OP_DISTILL, OP_FEATURE_BWD, OP_BWD_RECOMPUTE,
    lizard_attn_fwd_continue_feat, lizard_attn_decode_step_feat, lizard_hedgehog_fwd, lizard_hedgehog_bwd,
    hedgehog_fwd, hedgehog_bwd, lizard_attn_fwd_feat, lizard_attn_bwd_feat, fwd_feat, bwd_feat,
    lizard_distill_mse, distill_mse, lizard_gate_proj_fwd, lizard_gate_proj_bwd, gate_proj_workspace,
    gate_proj_fwd, gate_proj_bwd,
)
