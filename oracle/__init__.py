"""Float64 CPU oracle for the row-wise GRPO logits pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never imports, links or calls it, and it shares no code with the HIP path.
"""
from .grpo import (  # noqa: F401
    decode_bf16, to_f64, log_softmax_stats, selective_log_softmax,
    selective_log_softmax_bwd, entropy_from_logits, ppo_clip_terms, k3,
    grpo_forward, grpo_dlogp, dlogits_from_dlogp, grpo_backward,
    fused_linear_grpo, fused_linear_loss,
    entropy_from_logits_bwd, group_advantages, loss_weights,
)
