"""Row-wise GRPO logits pass for MI355X (gfx950): HIP kernels behind a C ABI.

The functions below are thin ctypes bindings of ``libgrpo_rows.so`` (built by
``python -m rl_fine_tuning_row_amd.build``); PyTorch supplies device memory
and the HIP stream only.
"""
from ._lib import (  # noqa: F401
    GRPO_BF16, GRPO_F32, GRPO_FLAG_FORCE_DENSE, GRPO_SEQUENCE, GRPO_TOKEN, GrpoError,
    GrpoParams, LIB_PATH, entropy_from_logits, fused_linear_grpo_chunk,
    fused_linear_grpo_workspace_bytes, grpo_gemm_bf16, grpo_gemm_bf16_logits, grpo_logits_bwd,
    grpo_logits_fwd, grpo_logits_fwd_bwd, header_functions, logits_partials,
    lib, selective_log_softmax, selective_log_softmax_bwd,
    entropy_from_logits_bwd, grpo_group_advantages, grpo_loss_weights, GRPO_REDUCE,
    fused_linear_grpo_chunk_noalloc, NOALLOC_SCRATCH_BYTES,
)
