// aux.hip -- the steps either side of the row pass: group-relative
// advantages (before it) and the per-token weights of a loss reduction (the
// dloss the backward consumes).  Small, latency-bound kernels.
#include <hip/hip_runtime.h>

#include "grpo_rows.h"
#include "host_common.hpp"

using grpo::aligned;
using grpo::groups_per_launch;

namespace {

// One thread per group of G consecutive rewards.  Sums in fp64 so that the
// only fp32 rounding is the stored result.  A group whose rewards are all
// equal (or a group of one) gets exactly 0; a NaN reward makes its group NaN.
__global__ __launch_bounds__(256) void group_advantages_kernel(const float* __restrict__ rewards,
                                                               int64_t groups, int G, float eps,
                                                               int scale, float* __restrict__ adv) {
  const int64_t k = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (k >= groups) return;
  const float* r = rewards + k * G;
  float* a = adv + k * G;
  float hi = r[0], lo = r[0];
  double sum = 0.0;
  for (int i = 0; i < G; ++i) {
    const float x = r[i];
    hi = x > hi ? x : hi;
    lo = x < lo ? x : lo;
    sum += double(x);
  }
  if (hi == lo && sum == sum) {
    for (int i = 0; i < G; ++i) a[i] = 0.0f;
    return;
  }
  const double mean = sum / G;
  double ss = 0.0;
  for (int i = 0; i < G; ++i) {
    const double d = double(r[i]) - mean;
    ss += d * d;
  }
  const double den = scale ? sqrt(ss / (G - 1)) + double(eps) : 1.0;
  for (int i = 0; i < G; ++i) a[i] = float((double(r[i]) - mean) / den);
}

// token mean: one workgroup counts every kept token, then writes 1/count
__global__ __launch_bounds__(1024) void weights_token_kernel(const uint8_t* __restrict__ mask,
                                                             int64_t n, float* __restrict__ w) {
  __shared__ long long part[16];
  long long cnt = 0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) cnt += mask == nullptr ? 1 : (mask[i] != 0);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  long long tot = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) tot += part[k];
  const float v = float(1.0 / double(tot > 0 ? tot : 1));
  for (int64_t i = threadIdx.x; i < n; i += 1024)
    w[i] = (mask == nullptr || mask[i] != 0) ? v : 0.0f;
}

// per-sequence mean (1 / (n_b B)) or constant normaliser (1 / (B L)):
// one workgroup per sequence
__global__ __launch_bounds__(256) void weights_seq_kernel(const uint8_t* __restrict__ mask,
                                                          int64_t B, int L, int per_sequence,
                                                          int64_t b0, float* __restrict__ w) {
  const int64_t b = b0 + blockIdx.x;
  const uint8_t* m = mask == nullptr ? nullptr : mask + b * L;
  float v;
  if (per_sequence) {
    __shared__ int part[4];
    int cnt = 0;
    for (int t = threadIdx.x; t < L; t += 256) cnt += m == nullptr ? 1 : (m[t] != 0);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
    __syncthreads();
    const int n = part[0] + part[1] + part[2] + part[3];
    v = float(1.0 / (double(n > 0 ? n : 1) * double(B)));
  } else {
    v = float(1.0 / (double(B) * double(L)));
  }
  for (int t = threadIdx.x; t < L; t += 256)
    w[b * L + t] = (m == nullptr || m[t] != 0) ? v : 0.0f;
}

}  // namespace

extern "C" int grpo_group_advantages(const float* rewards, int64_t n, int64_t group_size,
                                     float eps, int scale, float* adv, void* stream) {
  if (n < 0 || group_size <= 0 || group_size > (int64_t(1) << 24) || n % group_size != 0 ||
      n > (int64_t(1) << 31))
    return GRPO_ERR_SHAPE;
  if (!(eps >= 0.0f) || (scale != 0 && scale != 1)) return GRPO_ERR_PARAM;
  if (n == 0) return GRPO_OK;
  if (rewards == nullptr || adv == nullptr) return GRPO_ERR_NULL;
  if (!aligned(rewards, 4) || !aligned(adv, 4)) return GRPO_ERR_ALIGN;
  const int64_t groups = n / group_size;
  hipLaunchKernelGGL(group_advantages_kernel, dim3(unsigned((groups + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), rewards, groups, int(group_size), eps,
                     scale, adv);
  return hipGetLastError() == hipSuccess ? GRPO_OK : GRPO_ERR_LAUNCH;
}

extern "C" int grpo_loss_weights(const uint8_t* mask, int64_t B, int64_t L, int reduction,
                                 float* dloss, void* stream) {
  if (B < 0 || L < 0 || L > (int64_t(1) << 30) || B > (int64_t(1) << 31)) return GRPO_ERR_SHAPE;
  if (reduction != GRPO_REDUCE_TOKEN && reduction != GRPO_REDUCE_SEQUENCE &&
      reduction != GRPO_REDUCE_CONSTANT)
    return GRPO_ERR_PARAM;
  if (B == 0 || L == 0) return GRPO_OK;
  if (dloss == nullptr) return GRPO_ERR_NULL;
  if (!aligned(dloss, 4)) return GRPO_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (reduction == GRPO_REDUCE_TOKEN)
    hipLaunchKernelGGL(weights_token_kernel, dim3(1), dim3(1024), 0, s, mask, B * L, dloss);
  else
    for (int64_t b0 = 0, step = groups_per_launch(256); b0 < B; b0 += step) {
      hipLaunchKernelGGL(weights_seq_kernel, dim3(unsigned(B - b0 < step ? B - b0 : step)),
                         dim3(256), 0, s, mask, B, int(L), reduction == GRPO_REDUCE_SEQUENCE ? 1 : 0,
                         b0, dloss);
      if (hipGetLastError() != hipSuccess) return GRPO_ERR_LAUNCH;
    }
  return hipGetLastError() == hipSuccess ? GRPO_OK : GRPO_ERR_LAUNCH;
}
