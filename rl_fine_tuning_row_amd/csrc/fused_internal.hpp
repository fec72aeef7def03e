// fused_internal.hpp -- the chunked fused-linear loss's steps, shared by its
// two C ABI entry points (caller workspace, and the static scratch of the
// entry point that allocates nothing).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "grpo_rows.h"

namespace grpo {

// Argument checks of fused_linear_grpo_chunk apart from the workspace.
int fused_chunk_check(const void* hidden, int64_t nseq, int64_t L, int64_t H, const void* weight,
                      int64_t V, const int64_t* ids, const float* old_logp, const float* ref_logp,
                      const float* adv, const uint8_t* mask, const float* dloss,
                      const grpo_params* p, float* loss_accum, float* grad_hidden,
                      float* grad_weight);

// Workspace bytes the chunk's steps use for R rows.
size_t fused_chunk_workspace(int64_t R, int64_t V, int64_t H);

// Enqueue the chunk's steps on `s` with the given workspace (at least
// fused_chunk_workspace bytes, 256-byte aligned; nothing in it needs to start
// zeroed: every step writes what a later one reads).  use_side_stream runs
// grad_weight's product on the library's per-device side stream (forked and
// joined through events made per call); false keeps everything on `s` and
// creates nothing.  Arguments already checked; nseq > 0.
int fused_chunk_run(const void* hidden, int64_t nseq, int64_t L, int64_t H, const void* weight,
                    int64_t V, const int64_t* ids, const float* old_logp, const float* ref_logp,
                    const float* adv, const float* dloss, const grpo_params* p,
                    float* loss_accum, float* grad_hidden, float* grad_weight, void* workspace,
                    hipStream_t s, bool use_side_stream);

}  // namespace grpo
