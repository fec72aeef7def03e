// fused_linear.hip -- one batch chunk of the chunked fused-linear GRPO loss.
//
// The LM-head input is processed one chunk of sequences at a time and the
// gradients of the chunk's hidden states and of the LM-head weight are taken
// during the forward and accumulated, so the whole batch's logits never
// exist ["Liger GRPO meets TRL" summary, detailed items 3 and 4].  Per chunk
// of R = nseq * L rows, all on the caller's stream:
//   1. z  = h W^T                 MFMA GEMM, fp32 [R, V] in the workspace
//   2. row forward on z           lse, logp, per-token loss (fp32 rows)
//   3. row backward on z          dz = g/T (onehot - p) as bf16 [R, V]
//   4. loss_accum += sum dloss * loss     (one workgroup, fixed order)
//   5. grad_hidden = dz W         MFMA GEMM split over V, partial sums reduced
//                                 in a fixed order (deterministic)
//   6. grad_weight += dz^T h      MFMA GEMM accumulating into fp32
// z stays fp32 so the per-token loss meets a 1e-5 relative bar; dz is
// rounded to bf16 before the two products (the matrix cores' input type).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "gemm_mfma.hpp"
#include "grpo_rows.h"
#include "host_common.hpp"
#include "row_core.hpp"
#include "rows_internal.hpp"

namespace grpo {
namespace {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t z_off, dz_off, logp_off, lse_off, loss_off, total;
  int splits;
};

// K-splits of grad_hidden = dz W so that the 256 x 256 tiles times the
// splits give at least two workgroups per CU.
int pick_splits(int64_t R, int64_t H) {
  const int64_t tiles = ((R + 255) / 256) * ((H + 255) / 256);
  int s = 1;
  while (tiles * s < 512 && s < 16) s *= 2;
  return s;
}

WsLayout ws_layout(int64_t R, int64_t V, int64_t H) {
  WsLayout w{};
  w.splits = pick_splits(R, H);
  const size_t zb = size_t(R) * size_t(V) * 4;
  const size_t part = w.splits > 1 ? size_t(w.splits) * size_t(R) * size_t(H) * 4 : 0;
  w.z_off = 0;  // z, later reused for the split-K partial sums
  w.dz_off = align256(std::max(zb, part));
  w.logp_off = w.dz_off + align256(size_t(R) * size_t(V) * 2);
  w.lse_off = w.logp_off + align256(size_t(R) * 4);
  w.loss_off = w.lse_off + align256(size_t(R) * 4);
  w.total = w.loss_off + align256(size_t(R) * 4);
  return w;
}

__global__ __launch_bounds__(1024) void weighted_sum_kernel(const float* __restrict__ loss,
                                                            const float* __restrict__ w, int n,
                                                            float* __restrict__ acc) {
  float s = 0.0f;
  for (int i = threadIdx.x; i < n; i += 1024) s += w[i] * loss[i];
  s = wave_sum(s);
  __shared__ float sh[16];
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += sh[k];
    *acc += t;
  }
}

// out[i] = sum_z part[z * stride + i], z in order; n is a multiple of 4
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int64_t n,
                                                            int64_t stride,
                                                            float* __restrict__ out) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float4 s = *reinterpret_cast<const float4*>(part + i);
  for (int z = 1; z < splits; ++z) {
    const float4 v = *reinterpret_cast<const float4*>(part + int64_t(z) * stride + i);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  *reinterpret_cast<float4*>(out + i) = s;
}

int check_fused(const void* hidden, int64_t nseq, int64_t L, int64_t H, const void* weight,
                int64_t V, const int64_t* ids, const float* old_logp, const float* ref_logp,
                const float* adv, const uint8_t* mask, const float* dloss, const grpo_params* p,
                float* loss_accum, float* grad_hidden, float* grad_weight, void* workspace) {
  if (nseq < 0 || L <= 0 || H <= 0 || V <= 0) return GRPO_ERR_SHAPE;
  if (H % 64 != 0 || H > 65536 || V % 8 != 0 || V > (int64_t(1) << 30)) return GRPO_ERR_SHAPE;
  if (nseq > (int64_t(1) << 30) / L) return GRPO_ERR_SHAPE;
  const int st = check_params(p);
  if (st != GRPO_OK) return st;
  if (p->level != GRPO_TOKEN || (p->flags & GRPO_FLAG_FORCE_DENSE)) return GRPO_ERR_PARAM;
  if (nseq == 0) return GRPO_OK;
  if (hidden == nullptr || weight == nullptr || ids == nullptr || old_logp == nullptr ||
      adv == nullptr || dloss == nullptr || loss_accum == nullptr || grad_hidden == nullptr ||
      grad_weight == nullptr || workspace == nullptr)
    return GRPO_ERR_NULL;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 256) ||
      !aligned(ids, 8) || !aligned(old_logp, 4) || !aligned(ref_logp, 4) || !aligned(adv, 4) ||
      !aligned(dloss, 4) || !aligned(loss_accum, 4) || !aligned(grad_hidden, 16) ||
      !aligned(grad_weight, 4))
    return GRPO_ERR_ALIGN;
  (void)mask;
  return GRPO_OK;
}

}  // namespace
}  // namespace grpo

using namespace grpo;

extern "C" size_t fused_linear_grpo_workspace_bytes(int64_t rows, int64_t V, int64_t H) {
  if (rows < 0 || V <= 0 || H <= 0 || rows > (int64_t(1) << 30)) return 0;
  return ws_layout(rows, V, H).total;
}

extern "C" int fused_linear_grpo_chunk(const void* hidden, int64_t nseq, int64_t L, int64_t H,
                                       const void* weight, int64_t V, const int64_t* ids,
                                       const float* old_logp, const float* ref_logp,
                                       const float* adv, const uint8_t* mask, const float* dloss,
                                       const grpo_params* p, float* loss_accum,
                                       float* grad_hidden, float* grad_weight, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  int st = check_fused(hidden, nseq, L, H, weight, V, ids, old_logp, ref_logp, adv, mask, dloss,
                       p, loss_accum, grad_hidden, grad_weight, workspace);
  if (st != GRPO_OK || nseq == 0) return st;
  const int64_t R = nseq * L;
  const WsLayout w = ws_layout(R, V, H);
  if (workspace_bytes < w.total) return GRPO_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  float* z = reinterpret_cast<float*>(base + w.z_off);
  uint16_t* dz = reinterpret_cast<uint16_t*>(base + w.dz_off);
  float* logp = reinterpret_cast<float*>(base + w.logp_off);
  float* lse = reinterpret_cast<float*>(base + w.lse_off);
  float* loss = reinterpret_cast<float*>(base + w.loss_off);
  const uint16_t* h = static_cast<const uint16_t*>(hidden);
  const uint16_t* W = static_cast<const uint16_t*>(weight);

  // 1. logits of the chunk
  GemmArgs g1{};
  g1.A = h;
  g1.lda = H;
  g1.B = W;
  g1.ldb = H;
  g1.C = z;
  g1.ldc = V;
  g1.M = int32_t(R);
  g1.N = int32_t(V);
  g1.K = int32_t(H);
  g1.k_per_split = int32_t(H);
  if (gemm_bf16(true, true, GEMM_STORE, g1, 1, s) != hipSuccess) return GRPO_ERR_LAUNCH;

  // 2. forward row pass on the fp32 logits
  FwdArgs fa{};
  fa.logits = z;
  fa.ld = V;
  fa.V = int32_t(V);
  fa.L = int32_t(L);
  fa.ids = ids;
  fa.old_logp = old_logp;
  fa.ref_logp = ref_logp;
  fa.adv = adv;
  fa.T = p->temperature;
  fa.c = kLog2e / p->temperature;
  fa.beta = p->beta;
  fa.lo = 1.0f - p->eps_low;
  fa.hi = 1.0f + p->eps_high;
  fa.mode = FWD_GRPO;
  fa.level = GRPO_TOKEN;
  fa.loss = loss;
  fa.logp = logp;
  fa.lse = lse;
  st = launch_fwd(fa, GRPO_F32, R, false, s);
  if (st != GRPO_OK) return st;

  // 3. backward row pass: bf16 dz
  BwdArgs ba{};
  ba.logits = z;
  ba.ld = V;
  ba.dlogits = dz;
  ba.ld_out = V;
  ba.V = int32_t(V);
  ba.L = int32_t(L);
  ba.ids = ids;
  ba.old_logp = old_logp;
  ba.ref_logp = ref_logp;
  ba.adv = adv;
  ba.mask = mask;
  ba.logp = logp;
  ba.lse = lse;
  ba.dloss = dloss;
  ba.T = fa.T;
  ba.c = fa.c;
  ba.beta = fa.beta;
  ba.lo = fa.lo;
  ba.hi = fa.hi;
  ba.mode = BWD_GRPO;
  ba.level = GRPO_TOKEN;
  st = launch_bwd_f32_to_bf16(ba, R, s);
  if (st != GRPO_OK) return st;

  // 4. loss of the chunk
  hipLaunchKernelGGL(weighted_sum_kernel, dim3(1), dim3(1024), 0, s, loss, dloss, int(R),
                     loss_accum);
  if (hipGetLastError() != hipSuccess) return GRPO_ERR_LAUNCH;

  // 5. grad_hidden = dz W, split over V; partial sums reuse the z region
  GemmArgs g2{};
  g2.A = dz;
  g2.lda = V;
  g2.B = W;
  g2.ldb = H;
  g2.M = int32_t(R);
  g2.N = int32_t(H);
  g2.K = int32_t(V);
  const int64_t per = (V + w.splits - 1) / w.splits;
  g2.k_per_split = int32_t(((per + 63) / 64) * 64);
  g2.split_stride = R * H;
  g2.C = w.splits > 1 ? z : grad_hidden;
  g2.ldc = H;
  if (gemm_bf16(true, false, GEMM_STORE, g2, w.splits, s) != hipSuccess) return GRPO_ERR_LAUNCH;
  if (w.splits > 1) {
    const int64_t n = R * H;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(unsigned((n / 4 + 255) / 256)), dim3(256), 0,
                       s, z, w.splits, n, n, grad_hidden);
    if (hipGetLastError() != hipSuccess) return GRPO_ERR_LAUNCH;
  }

  // 6. grad_weight += dz^T h
  GemmArgs g3{};
  g3.A = dz;
  g3.lda = V;
  g3.B = h;
  g3.ldb = H;
  g3.C = grad_weight;
  g3.ldc = H;
  g3.M = int32_t(V);
  g3.N = int32_t(H);
  g3.K = int32_t(R);
  g3.k_per_split = int32_t(((R + 63) / 64) * 64);
  if (gemm_bf16(false, false, GEMM_ACCUM, g3, 1, s) != hipSuccess) return GRPO_ERR_LAUNCH;
  return GRPO_OK;
}
