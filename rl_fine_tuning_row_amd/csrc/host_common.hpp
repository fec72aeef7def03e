// host_common.hpp -- host-side argument checks shared by the entry points.
// Plain C++: no device calls, so every check runs before anything is enqueued.
#pragma once

#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "grpo_rows.h"

namespace grpo {

constexpr int64_t kMaxV = int64_t(1) << 26;        // row length limit (int32 lane indexing)
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1; // rows per call

// A dispatch packet holds each grid dimension in work-items as a 32-bit
// number, so one launch covers at most 2^32 - 1 work-items (4194303
// workgroups of 1024 lanes).  Launchers of grids that can be larger (one or
// more workgroups per row, per sequence or per hidden row) cut them into
// slices of whole workgroups and pass each slice's first index.
constexpr int64_t kMaxLaunchItems = (int64_t(1) << 32) - 1;
inline int64_t groups_per_launch(int threads) { return kMaxLaunchItems / threads; }

inline int elem_size(int dtype) { return dtype == GRPO_BF16 ? 2 : 4; }

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int check_dtype(int dtype) {
  return (dtype == GRPO_F32 || dtype == GRPO_BF16) ? GRPO_OK : GRPO_ERR_DTYPE;
}

// logits-like matrix [rows, ld] with V used columns
inline int check_matrix(const void* ptr, int dtype, int64_t rows, int64_t V, int64_t ld) {
  int st = check_dtype(dtype);
  if (st != GRPO_OK) return st;
  if (rows < 0 || rows > kMaxRows || V <= 0 || V > kMaxV) return GRPO_ERR_SHAPE;
  if (ld < V) return GRPO_ERR_STRIDE;
  if (rows > 0 && ptr == nullptr) return GRPO_ERR_NULL;
  if (!aligned(ptr, elem_size(dtype))) return GRPO_ERR_ALIGN;
  return GRPO_OK;
}

inline int check_temperature(float T) {
  return (std::isfinite(T) && T > 0.0f) ? GRPO_OK : GRPO_ERR_PARAM;
}

inline int check_params(const grpo_params* p) {
  if (p == nullptr) return GRPO_ERR_NULL;
  if (check_temperature(p->temperature) != GRPO_OK) return GRPO_ERR_PARAM;
  if (!std::isfinite(p->beta) || p->beta < 0.0f) return GRPO_ERR_PARAM;
  if (!std::isfinite(p->eps_low) || p->eps_low < 0.0f || p->eps_low >= 1.0f) return GRPO_ERR_PARAM;
  if (!std::isfinite(p->eps_high) || p->eps_high < 0.0f) return GRPO_ERR_PARAM;
  if (p->level != GRPO_TOKEN && p->level != GRPO_SEQUENCE) return GRPO_ERR_PARAM;
  if ((p->flags & ~uint32_t(GRPO_FLAG_FORCE_DENSE)) != 0) return GRPO_ERR_PARAM;
  return GRPO_OK;
}

// optional launch shape overrides "WG,UNROLL" for tuning sweeps:
// GRPO_ROWS_FWD_LAUNCH (forward-type kernels), GRPO_ROWS_BWD_LAUNCH
// (backward-type kernels), GRPO_ROWS_LAUNCH (both).  Unset: built-in policy.
struct LaunchOverride {
  int wg = 0, unroll = 0;
};
inline LaunchOverride parse_launch(const char* e) {
  LaunchOverride r;
  if (e != nullptr) {
    char* end = nullptr;
    r.wg = int(std::strtol(e, &end, 10));
    if (end != nullptr && *end == ',') r.unroll = int(std::strtol(end + 1, nullptr, 10));
  }
  return r;
}
inline LaunchOverride launch_override(int which) {
  static const LaunchOverride both = parse_launch(std::getenv("GRPO_ROWS_LAUNCH"));
  static const LaunchOverride fwd = parse_launch(std::getenv("GRPO_ROWS_FWD_LAUNCH"));
  static const LaunchOverride bwd = parse_launch(std::getenv("GRPO_ROWS_BWD_LAUNCH"));
  const LaunchOverride& o = which == 0 ? fwd : bwd;
  return (o.wg > 0) ? o : both;
}

}  // namespace grpo
