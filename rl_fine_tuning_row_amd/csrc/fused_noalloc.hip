// fused_noalloc.hip -- fused_linear_grpo_chunk_noalloc: the chunked
// fused-linear loss for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// It runs the same steps and kernels as fused_linear_grpo_chunk, with the
// workspace in a file-scope device array of kScratchBytes instead of a
// caller buffer, and every step on the caller's stream (the other entry
// point's side stream and per-call events are objects the runtime would
// create).  The array lives in this file's code object, which has no
// kernels of its own, so a process pays for it only once it calls this
// entry point; each device then holds its own copy until the process ends.
//
// In host code `scratch` is only a stand-in symbol: its device address is
// taken once per device with hipGetSymbolAddress and that pointer, never the
// name, is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fused_internal.hpp"
#include "grpo_rows.h"

namespace {

// 384 MiB: the chunk workspace of one 1024-token sequence at a
// 151936-entry vocabulary and H = 1024 (about 363 MiB: its bf16 logits, the
// split-K partial sums and the compacted hidden states), 0.13% of the
// device's 288 GB.
constexpr size_t kScratchBytes = size_t(384) << 20;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// The scratch array's device address on the current device (taken on the
// first call there), or nullptr if the runtime cannot give it.
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" int fused_linear_grpo_chunk_noalloc(const void* hidden, int64_t nseq, int64_t L,
                                               int64_t H, const void* weight, int64_t V,
                                               const int64_t* ids, const float* old_logp,
                                               const float* ref_logp, const float* adv,
                                               const uint8_t* mask, const float* dloss,
                                               const grpo_params* p, float* loss_accum,
                                               float* grad_hidden, float* grad_weight,
                                               void* stream) {
  int st = grpo::fused_chunk_check(hidden, nseq, L, H, weight, V, ids, old_logp, ref_logp, adv,
                                   mask, dloss, p, loss_accum, grad_hidden, grad_weight);
  if (st != GRPO_OK || nseq == 0) return st;
  if (grpo::fused_chunk_workspace(nseq * L, V, H) > kScratchBytes) return GRPO_ERR_SCRATCH;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return GRPO_ERR_LAUNCH;
  return grpo::fused_chunk_run(hidden, nseq, L, H, weight, V, ids, old_logp, ref_logp, adv, dloss,
                               p, loss_accum, grad_hidden, grad_weight, ws,
                               static_cast<hipStream_t>(stream), false);
}
