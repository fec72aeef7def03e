// fused_linear.hip -- one batch chunk of the chunked fused-linear GRPO loss.
//
// The LM-head input is processed one chunk of sequences at a time and the
// gradients of the chunk's hidden states and of the LM-head weight are taken
// during the forward and accumulated, so the whole batch's logits never
// exist ["Liger GRPO meets TRL" summary, detailed items 3 and 4].  Per chunk
// of R = nseq * L rows, all on the caller's stream:
//   0. compaction                 the rows whose weight dloss is nonzero, in
//                                 order (one workgroup), their h rows and
//                                 per-row inputs gathered; Rc of them
//   1. z  = h_c W^T               MFMA GEMM; its epilogue keeps the fp32
//                                 accumulators for each row's softmax
//                                 statistics over every 128-column half-tile
//                                 and the target logit, and writes z as
//                                 bf16 [Rc, V] to the workspace
//   2. row forward                the partial statistics merged in a fixed
//                                 order: lse, logp, per-token loss (fp32)
//   3. row backward on bf16 z     dz = g/T (onehot - p) as bf16, in place
//   4. loss_accum += sum dloss * loss     (one workgroup, fixed order)
//   5. grad_hidden = dz W         MFMA GEMM split over V, partial sums reduced
//                                 in a fixed order (deterministic) and
//                                 scattered back; dropped rows get 0
//   6. grad_weight += dz^T h_c    MFMA GEMM accumulating into fp32, on a
//                                 side stream beside 5, joined before return
// A row with dloss = 0 (padding, a masked token) adds 0 to the loss and its
// dlogp, hence its dz row and its grad_hidden row, is 0: skipping it is the
// zero-gradient skip of the logits backward ["[Liger-Kernel] LinkedIn
// Liger-Kernel GRPO Loss Backward optimisation", Why is this good] carried
// into the chunked products.  (Non-finite inputs on such a row are dropped
// with it instead of propagating through 0 * inf.)  Rc is only known on the
// device: every later launch is sized for R and reads Rc there.
// The statistics, logp and loss come from the fp32 accumulators, so the
// per-token loss meets a 1e-5 relative bar; the backward's softmax reads the
// bf16 copy of z (the model's logits dtype), and dz is bf16 for the two
// products (the matrix cores' input type).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "fused_internal.hpp"
#include "gemm_mfma.hpp"
#include "grpo_rows.h"
#include "host_common.hpp"
#include "row_core.hpp"
#include "rows_internal.hpp"

namespace grpo {
namespace {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// A second stream per device (default priority, created on first use, kept
// for the process) for grad_weight's product, which runs beside
// grad_hidden's: both only read dz, and the split-K product leaves CUs idle
// in its last round that the other product's tiles then fill.  Each call
// forks and joins through events of its own, so concurrent callers stay
// ordered; their side work just shares the stream.  nullptr when it cannot be
// made (the products then run one after the other on the caller's stream).
hipStream_t side_stream() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static hipStream_t per[kMaxDevices] = {};
  static bool tried[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!tried[dev]) {
    tried[dev] = true;
    hipStream_t st = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess) per[dev] = st;
    else (void)hipGetLastError();
  }
  return per[dev];
}

struct WsLayout {
  size_t z_off, part_off, zy_off, logp_off, lse_off, loss_off;
  size_t map_off, pos_off, cnt_off, hc_off, ids_off, old_off, ref_off, adv_off, w_off;
  size_t total;
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
  const size_t stats = size_t(2) * size_t(logits_halves(V)) * size_t(R) * 4;
  const size_t splitk = size_t(w.splits) * size_t(R) * size_t(H) * 4;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  // z and h_c hold the kept rows rounded up to 64: grad_weight's product runs
  // over that many rows, the ones past the kept count zeroed, so that its K
  // steps are all whole (a partial last K step takes the masked path in
  // every tile: 8-10% slower)
  const int64_t Rp = (R + 63) / 64 * 64;
  w.z_off = take(size_t(Rp) * size_t(V) * 2);  // bf16 z, then dz in place
  w.part_off = take(std::max(stats, splitk));  // row statistics, then split-K partial sums
  w.zy_off = take(size_t(R) * 4);
  w.logp_off = take(size_t(R) * 4);
  w.lse_off = take(size_t(R) * 4);
  w.loss_off = take(size_t(R) * 4);
  w.map_off = take(size_t(R) * 4);
  w.pos_off = take(size_t(R) * 4);
  w.cnt_off = take(8);  // kept rows, then that count rounded up to 64
  w.hc_off = take(size_t(Rp) * size_t(H) * 2);
  w.ids_off = take(size_t(R) * 8);
  w.old_off = take(size_t(R) * 4);
  w.ref_off = take(size_t(R) * 4);
  w.adv_off = take(size_t(R) * 4);
  w.w_off = take(size_t(R) * 4);
  w.total = o;
  return w;
}

// Compaction of the rows with nonzero weight, in order, by one workgroup:
// map[i] = original row of compact row i, pos[r] = compact index of row r or
// -1, *count = number kept; the kept rows' per-row inputs are gathered
// (advantage per row, so the compact problem has one token per "sequence").
// NaN weights are kept (NaN != 0).
__global__ __launch_bounds__(1024) void compact_rows_kernel(
    int R, int L, const float* __restrict__ dloss, const int64_t* __restrict__ ids,
    const float* __restrict__ old_logp, const float* __restrict__ ref_logp,
    const float* __restrict__ adv, int32_t* __restrict__ map, int32_t* __restrict__ pos,
    int32_t* __restrict__ count, int64_t* __restrict__ ids_c, float* __restrict__ old_c,
    float* __restrict__ ref_c, float* __restrict__ adv_c, float* __restrict__ w_c) {
  __shared__ int wave_tot[16];
  __shared__ int base_sh;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) base_sh = 0;
  __syncthreads();
  for (int r0 = 0; r0 < R; r0 += 1024) {
    const int r = r0 + t;
    const float w = r < R ? dloss[r] : 0.0f;
    const bool keep = r < R && w != 0.0f;
    const uint64_t bal = __ballot(keep);
    const int below = __popcll(bal & ((uint64_t(1) << lane) - 1));
    if (lane == 0) wave_tot[wave] = __popcll(bal);
    __syncthreads();
    int off = base_sh;
    for (int k = 0; k < wave; ++k) off += wave_tot[k];
    const int i = off + below;
    if (r < R) pos[r] = keep ? i : -1;
    if (keep) {
      map[i] = r;
      ids_c[i] = ids[r];
      old_c[i] = old_logp[r];
      ref_c[i] = ref_logp != nullptr ? ref_logp[r] : 0.0f;
      adv_c[i] = adv[r / L];
      w_c[i] = w;
    }
    __syncthreads();  // every lane has read base_sh and wave_tot
    if (t == 0) {
      int tot = 0;
      for (int k = 0; k < 16; ++k) tot += wave_tot[k];
      base_sh += tot;
    }
    __syncthreads();
  }
  if (t == 0) {
    count[0] = base_sh;
    count[1] = (base_sh + 63) / 64 * 64;
  }
}

// Zero rows [count[0], count[1]) of z (ldz columns, the first V written) and
// of h_c (H columns): the rows grad_weight's product adds past the kept
// ones.  One workgroup per row, at most 63 rows; V and H multiples of 8.
__global__ __launch_bounds__(1024) void zero_pad_rows_kernel(const int32_t* __restrict__ count,
                                                             uint16_t* __restrict__ z,
                                                             int64_t ldz, int V,
                                                             uint16_t* __restrict__ h_c, int H) {
  const int64_t i = int64_t(count[0]) + blockIdx.x;
  if (i >= count[1]) return;
  const uint4 zero = {0u, 0u, 0u, 0u};
  uint4* zr = reinterpret_cast<uint4*>(z + i * ldz);
  for (int v = threadIdx.x; v < V / 8; v += 1024) zr[v] = zero;
  uint4* hr = reinterpret_cast<uint4*>(h_c + i * H);
  for (int v = threadIdx.x; v < H / 8; v += 1024) hr[v] = zero;
}

// h_c[i] = h[map[i]] for the kept rows; one workgroup per compact row,
// H % 8 == 0 (16-byte vectors)
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ h, int H,
                                                          const int32_t* __restrict__ map,
                                                          const int32_t* __restrict__ count,
                                                          int64_t i0, uint16_t* __restrict__ h_c) {
  const int64_t i = i0 + blockIdx.x;
  if (i >= *count) return;
  const uint4* src = reinterpret_cast<const uint4*>(h + int64_t(map[i]) * H);
  uint4* dst = reinterpret_cast<uint4*>(h_c + int64_t(i) * H);
  for (int v = threadIdx.x; v < H / 8; v += 256) dst[v] = src[v];
}

__global__ __launch_bounds__(1024) void weighted_sum_kernel(const float* __restrict__ loss,
                                                            const float* __restrict__ w,
                                                            const int32_t* __restrict__ count,
                                                            float* __restrict__ acc) {
  const int n = *count;
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

// grad_hidden row r = sum over splits z (in order) of the partial rows of its
// compact index pos[r], or 0 for a dropped row; H % 4 == 0
__global__ __launch_bounds__(256) void splitk_scatter_kernel(const float* __restrict__ part,
                                                             int splits, int64_t stride,
                                                             const int32_t* __restrict__ pos,
                                                             int64_t R, int H, int64_t e0,
                                                             float* __restrict__ out) {
  const int64_t e = e0 + (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e >= R * H) return;
  const int64_t r = e / H;
  const int c = int(e % H);
  const int p = pos[r];
  float4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  if (p >= 0) {
    const int64_t i = int64_t(p) * H + c;
    s = *reinterpret_cast<const float4*>(part + i);
    for (int z = 1; z < splits; ++z) {
      const float4 v = *reinterpret_cast<const float4*>(part + int64_t(z) * stride + i);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
  }
  *reinterpret_cast<float4*>(out + e) = s;
}

int check_fused(const void* hidden, int64_t nseq, int64_t L, int64_t H, const void* weight,
                int64_t V, const int64_t* ids, const float* old_logp, const float* ref_logp,
                const float* adv, const uint8_t* mask, const float* dloss, const grpo_params* p,
                float* loss_accum, float* grad_hidden, float* grad_weight, void* workspace) {
  if (nseq < 0 || L <= 0 || H <= 0 || V <= 0) return GRPO_ERR_SHAPE;
  if (H % 64 != 0 || H > 65536 || V % 8 != 0 || V > (int64_t(1) << 30)) return GRPO_ERR_SHAPE;
  if (nseq > (int64_t(1) << 30) / L) return GRPO_ERR_SHAPE;
  {
    // launch sizes: each product's tile grid (128 x 128 tiles at the
    // smallest, 256 lanes each; K-splits go in the second grid dimension)
    // must fit one dispatch's 32-bit work-item count
    const int64_t R = nseq * L;
    const int64_t lim = groups_per_launch(256);
    if (((R + 127) / 128) * ((V + 127) / 128) > lim) return GRPO_ERR_SHAPE;
    if (((V + 127) / 128) * ((H + 127) / 128) > lim) return GRPO_ERR_SHAPE;
    if (((R + 127) / 128) * ((H + 127) / 128) > lim) return GRPO_ERR_SHAPE;
  }
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

namespace grpo {

int fused_chunk_check(const void* hidden, int64_t nseq, int64_t L, int64_t H, const void* weight,
                      int64_t V, const int64_t* ids, const float* old_logp, const float* ref_logp,
                      const float* adv, const uint8_t* mask, const float* dloss,
                      const grpo_params* p, float* loss_accum, float* grad_hidden,
                      float* grad_weight) {
  // the workspace is checked by the caller (a buffer of its own, or the
  // no-alloc entry point's static scratch); any non-null stand-in passes here
  alignas(256) static char placeholder[1];
  return check_fused(hidden, nseq, L, H, weight, V, ids, old_logp, ref_logp, adv, mask, dloss, p,
                     loss_accum, grad_hidden, grad_weight, placeholder);
}

size_t fused_chunk_workspace(int64_t R, int64_t V, int64_t H) { return ws_layout(R, V, H).total; }

int fused_chunk_run(const void* hidden, int64_t nseq, int64_t L, int64_t H, const void* weight,
                    int64_t V, const int64_t* ids, const float* old_logp, const float* ref_logp,
                    const float* adv, const float* dloss, const grpo_params* p,
                    float* loss_accum, float* grad_hidden, float* grad_weight, void* workspace,
                    hipStream_t s, bool use_side_stream) {
  int st = GRPO_OK;
  const int64_t R = nseq * L;
  const WsLayout w = ws_layout(R, V, H);
  char* base = static_cast<char*>(workspace);
  uint16_t* z = reinterpret_cast<uint16_t*>(base + w.z_off);
  uint16_t* dz = z;  // the backward overwrites z in place
  float* part = reinterpret_cast<float*>(base + w.part_off);
  float* zy = reinterpret_cast<float*>(base + w.zy_off);
  float* logp = reinterpret_cast<float*>(base + w.logp_off);
  float* lse = reinterpret_cast<float*>(base + w.lse_off);
  float* loss = reinterpret_cast<float*>(base + w.loss_off);
  int32_t* map = reinterpret_cast<int32_t*>(base + w.map_off);
  int32_t* pos = reinterpret_cast<int32_t*>(base + w.pos_off);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + w.cnt_off);
  uint16_t* h_c = reinterpret_cast<uint16_t*>(base + w.hc_off);
  int64_t* ids_c = reinterpret_cast<int64_t*>(base + w.ids_off);
  float* old_c = reinterpret_cast<float*>(base + w.old_off);
  float* ref_c = reinterpret_cast<float*>(base + w.ref_off);
  float* adv_c = reinterpret_cast<float*>(base + w.adv_off);
  float* w_c = reinterpret_cast<float*>(base + w.w_off);
  const uint16_t* h = static_cast<const uint16_t*>(hidden);
  const uint16_t* W = static_cast<const uint16_t*>(weight);

  // 0. the rows that carry weight, and their inputs
  hipLaunchKernelGGL(compact_rows_kernel, dim3(1), dim3(1024), 0, s, int(R), int(L), dloss, ids,
                     old_logp, ref_logp, adv, map, pos, cnt, ids_c, old_c, ref_c, adv_c, w_c);
  for (int64_t i0 = 0, step = groups_per_launch(256); i0 < R; i0 += step)
    hipLaunchKernelGGL(gather_rows_kernel, dim3(unsigned(R - i0 < step ? R - i0 : step)), dim3(256),
                       0, s, h, int(H), map, cnt, i0, h_c);
  hipLaunchKernelGGL(zero_pad_rows_kernel, dim3(63), dim3(1024), 0, s, cnt, z, int64_t(V), int(V),
                     h_c, int(H));
  if (hipGetLastError() != hipSuccess) return GRPO_ERR_LAUNCH;

  // 1. logits of the kept rows: bf16 z, row statistics and target logits
  const float cscale = kLog2e / p->temperature;
  GemmArgs g1{};
  g1.A = h_c;
  g1.lda = H;
  g1.B = W;
  g1.ldb = H;
  g1.ldc = V;
  g1.M = int32_t(R);
  g1.N = int32_t(V);
  g1.K = int32_t(H);
  g1.k_per_split = int32_t(H);
  g1.dev_m = cnt;
  g1.z16 = z;
  g1.stat = part;
  g1.stat_ld = R;
  g1.ids = ids_c;
  g1.zy = zy;
  g1.cscale = cscale;
  if (gemm_bf16_logits(g1, s) != hipSuccess) return GRPO_ERR_LAUNCH;

  // 2. forward from the statistics (compact rows: one token per "sequence")
  FwdArgs fa{};
  fa.logits = nullptr;
  fa.ld = V;
  fa.V = int32_t(V);
  fa.L = 1;
  fa.ids = ids_c;
  fa.old_logp = old_c;
  fa.ref_logp = ref_logp != nullptr ? ref_c : nullptr;
  fa.adv = adv_c;
  fa.T = p->temperature;
  fa.c = cscale;
  fa.beta = p->beta;
  fa.lo = 1.0f - p->eps_low;
  fa.hi = 1.0f + p->eps_high;
  fa.mode = FWD_GRPO;
  fa.level = GRPO_TOKEN;
  fa.loss = loss;
  fa.logp = logp;
  fa.lse = lse;
  fa.dev_rows = cnt;
  st = launch_fwd_partials(fa, part, logits_halves(V), R, zy, R, s);
  if (st != GRPO_OK) return st;

  // 3. backward row pass: bf16 dz over bf16 z, in place
  BwdArgs ba{};
  ba.logits = z;
  ba.ld = V;
  ba.dlogits = dz;
  ba.ld_out = V;
  ba.V = int32_t(V);
  ba.L = 1;
  ba.ids = ids_c;
  ba.old_logp = old_c;
  ba.ref_logp = fa.ref_logp;
  ba.adv = adv_c;
  ba.mask = nullptr;
  ba.logp = logp;
  ba.lse = lse;
  ba.dloss = w_c;
  ba.T = fa.T;
  ba.c = fa.c;
  ba.beta = fa.beta;
  ba.lo = fa.lo;
  ba.hi = fa.hi;
  ba.mode = BWD_GRPO;
  ba.level = GRPO_TOKEN;
  ba.dev_rows = cnt;
  st = launch_bwd(ba, GRPO_BF16, R, s);
  if (st != GRPO_OK) return st;

  // 4. loss of the chunk
  hipLaunchKernelGGL(weighted_sum_kernel, dim3(1), dim3(1024), 0, s, loss, w_c, cnt, loss_accum);
  if (hipGetLastError() != hipSuccess) return GRPO_ERR_LAUNCH;

  // 5./6. the two gradient products, grad_weight's on the side stream
  hipStream_t s3 = s;
  hipEvent_t fork = nullptr, join = nullptr;
  if (hipStream_t side = use_side_stream ? side_stream() : nullptr) {
    if (hipEventCreateWithFlags(&fork, hipEventDisableTiming) == hipSuccess &&
        hipEventCreateWithFlags(&join, hipEventDisableTiming) == hipSuccess &&
        hipEventRecord(fork, s) == hipSuccess && hipStreamWaitEvent(side, fork, 0) == hipSuccess) {
      s3 = side;
    } else {
      (void)hipGetLastError();
    }
  }
  int status = GRPO_OK;

  // 6. grad_weight += dz^T h_c over the kept rows
  GemmArgs g3{};
  g3.A = dz;
  g3.lda = V;
  g3.B = h_c;
  g3.ldb = H;
  g3.C = grad_weight;
  g3.ldc = H;
  g3.M = int32_t(V);
  g3.N = int32_t(H);
  g3.K = int32_t((R + 63) / 64 * 64);
  g3.k_per_split = g3.K;
  g3.dev_k = cnt + 1;  // the kept rows rounded up to 64 (the extra rows are zero)
  if (gemm_bf16(false, false, GEMM_ACCUM, g3, 1, s3) != hipSuccess) status = GRPO_ERR_LAUNCH;

  // 5. grad_hidden = dz W, split over V into partial sums (the statistics' region),
  //    reduced in order and scattered to the original rows
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
  g2.C = part;
  g2.ldc = H;
  g2.dev_m = cnt;
  if (status == GRPO_OK && gemm_bf16(true, false, GEMM_STORE, g2, w.splits, s) != hipSuccess)
    status = GRPO_ERR_LAUNCH;
  if (status == GRPO_OK) {
    const int64_t n = R * H;
    const int64_t groups = (n / 4 + 255) / 256, step = groups_per_launch(256);
    for (int64_t g0 = 0; g0 < groups && status == GRPO_OK; g0 += step) {
      hipLaunchKernelGGL(splitk_scatter_kernel,
                         dim3(unsigned(groups - g0 < step ? groups - g0 : step)), dim3(256), 0, s,
                         part, w.splits, n, pos, R, int(H), g0 * 1024, grad_hidden);
      if (hipGetLastError() != hipSuccess) status = GRPO_ERR_LAUNCH;
    }
  }
  // the caller's stream waits for the side stream before anything after this
  // call (also after a failed launch: nothing may stay behind unordered)
  if (s3 != s && (hipEventRecord(join, s3) != hipSuccess || hipStreamWaitEvent(s, join, 0) != hipSuccess))
    status = GRPO_ERR_LAUNCH;
  if (fork != nullptr) (void)hipEventDestroy(fork);
  if (join != nullptr) (void)hipEventDestroy(join);
  return status;
}

}  // namespace grpo

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
  if (workspace_bytes < ws_layout(nseq * L, V, H).total) return GRPO_ERR_WORKSPACE;
  return fused_chunk_run(hidden, nseq, L, H, weight, V, ids, old_logp, ref_logp, adv, dloss, p,
                         loss_accum, grad_hidden, grad_weight, workspace,
                         static_cast<hipStream_t>(stream), true);
}
