"""fp64 CPU oracle for the chunked GRPO path.  Test infrastructure only."""
from .grpo_oracle import (  # noqa: F401
    cross_entropy_loss_and_grad,
    grad_rows,
    group_advantages,
    grpo_loss_and_grad,
    grpo_loss_from_logp,
    grpo_token_terms,
    logit_map,
    logits,
    logp_backward,
    selective_log_softmax,
    sequence_of_token,
    token_weights,
    widen,
)
