"""Chunked GRPO log-probabilities, loss and dL/dH on MI355X (gfx950).

The computation lives in the HIP library built from ``csrc/`` (C ABI in
include/grpo.h); ``grpo`` is its thin ctypes binding.
"""
from .grpo import (  # noqa: F401
    GRPO_BF16,
    GRPO_F32,
    GRPO_WS_HOST_H,
    GrpoError,
    Offload,
    Timer,
    grpo_advantages,
    grpo_ce_loss_fwd_bwd,
    grpo_debug_token_index,
    grpo_logp_bwd,
    grpo_logp_bwd_offload,
    grpo_logp_fwd,
    grpo_logp_fwd_offload,
    grpo_loss_fwd_bwd,
    grpo_loss_fwd_bwd_static,
    grpo_plan_info,
    grpo_workspace_bytes,
    lib,
)
