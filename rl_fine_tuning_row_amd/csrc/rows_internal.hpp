// rows_internal.hpp -- argument blocks and launchers of the row kernels,
// shared by the C ABI entry points and the fused-linear path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grpo {

enum FwdMode : int32_t { FWD_GRPO = 0, FWD_ENTROPY = 1, FWD_LSM = 2 };
enum BwdMode : int32_t { BWD_GRPO = 0, BWD_LSM = 1, BWD_ENTROPY = 2 };

struct FwdArgs {
  const void* logits;
  int64_t ld;
  int32_t V;
  int32_t L;  // tokens per sequence (GRPO); 1 otherwise
  const int64_t* ids;
  const float* old_logp;
  const float* ref_logp;
  const float* adv;
  float T, c, beta, lo, hi;
  int32_t mode, level;
  float* loss;
  float* logp;
  float* lse;
  float* entropy;
  float* kl;
  uint8_t* is_clipped;
  float* gathered;
  int32_t* err_count;
  const int32_t* dev_rows;  // nullable: rows at or past *dev_rows are skipped
  int64_t row0;             // first row of this launch (set by the launchers)
};

struct BwdArgs {
  const void* logits;
  int64_t ld;
  void* dlogits;
  int64_t ld_out;
  int32_t V;
  int32_t L;
  const int64_t* ids;
  const float* old_logp;
  const float* ref_logp;
  const float* adv;
  const uint8_t* mask;
  const float* logp;
  const float* lse;
  const float* seq_ratio;
  const float* dloss;    // grad_logp in BWD_LSM mode, grad_entropy in BWD_ENTROPY
  const float* entropy;  // BWD_ENTROPY: the rows' entropies H
  float T, c, beta, lo, hi;
  int32_t mode, level, force_dense;
  uint8_t* zero_row;
  const int32_t* dev_rows;  // nullable: rows at or past *dev_rows are skipped
  int32_t nchunk;           // workgroups per row (set by the launchers, >= 1)
  int64_t row0;             // first row of this launch (set by the launchers)
};

struct SeqArgs {
  int32_t L;
  const float* logp;
  const float* old_logp;
  const uint8_t* mask;
  const float* adv;
  float lo, hi;
  float* loss;
  uint8_t* is_clipped;
  float* seq_ratio;
  int64_t b0;  // first sequence of this launch
};

// Launch the forward-type row kernel (GRPO / entropy / selective
// log-softmax, by a.mode) over `rows` rows of `dtype` logits.
int launch_fwd(const FwdArgs& a, int dtype, int64_t rows, bool need_t, hipStream_t s);
// Forward (FWD_GRPO, token level, no entropy) of rows whose softmax
// statistics come as P partials each (stat: m and s arrays of P * stat_ld
// floats, partial p of row r at p * stat_ld + r) and whose target logit is
// zy[r] (fp32).
int launch_fwd_partials(const FwdArgs& a, const float* stat, int P, int64_t stat_ld,
                        const float* zy, int64_t rows, hipStream_t s);
// Launch the backward row kernel; logits and dlogits of the same dtype.
int launch_bwd(const BwdArgs& a, int dtype, int64_t rows, hipStream_t s);
// Entropy backward (BWD_ENTROPY) on logits and dlogits of the same dtype.
int launch_bwd_entropy(const BwdArgs& a, int dtype, int64_t rows, hipStream_t s);

}  // namespace grpo
