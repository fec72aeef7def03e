// rows.hip -- HBM-bound row kernels and their C ABI entry points:
// grpo_logits_fwd, grpo_logits_bwd, entropy_from_logits,
// selective_log_softmax, selective_log_softmax_bwd.
//
// One workgroup per row (the backward splits rows into chunks of 8 or 64 KB,
// one workgroup each).  Lanes stream the row with 128-bit loads (8
// bf16 or 4 fp32 per lane), UNROLL vectors in flight per lane, fold each
// register tile into the online softmax state (row_core.hpp), reduce across
// the wave with lane shuffles and across waves through LDS, and lane 0 writes
// the per-row scalars.  The backward computes the row's dlogp first; it is
// the same in every lane (readfirstlane), so the all-zero early path
// [Liger-Kernel PR #1550 analysis, "Code analysis": the added
// ``if dlogp == 0.0`` early return] is a scalar branch that writes zeros
// without touching the logits.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "grpo_rows.h"
#include "host_common.hpp"
#include "row_core.hpp"
#include "rows_internal.hpp"

namespace grpo {

// ---------------------------------------------------------------------------
// forward: one pass over the row
// ---------------------------------------------------------------------------
// Values past the row end in a lane's registers: large, negative and finite,
// they add nothing to a max or a sum taken against a real element.
template <typename TIn> struct Fill;
template <> struct Fill<uint16_t> { static constexpr uint32_t bits = 0xF149F149u; };  // bf16 ~ -1e30
template <> struct Fill<float> { static constexpr uint32_t bits = 0xF149F2CAu; };     // -1e30f

template <typename TIn, int WG, int UNROLL, bool VEC, bool NEED_T, bool NTL>
__device__ __forceinline__ Stat scan_row(const TIn* __restrict__ row, int V, float c) {
  Stat st;
  stat_init(st);
  const int tid = threadIdx.x;
  if constexpr (VEC) {
    constexpr int VE = Vec<TIn>::N;
    const u32x4* __restrict__ rv = reinterpret_cast<const u32x4*>(row);
    const int nvec = V / VE;
    int i = tid;
    for (; i + (UNROLL - 1) * WG < nvec; i += UNROLL * WG) {
      u32x4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) v[u] = load16<NTL>(rv + i + u * WG);
      float x[UNROLL * VE];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) Vec<TIn>::unpack(v[u], x + u * VE);
      stat_tile<UNROLL * VE, NEED_T>(st, x, c);
    }
    if (i < nvec) {  // the last, partial batch: its loads issued at once
      const u32x4 fill = {Fill<TIn>::bits, Fill<TIn>::bits, Fill<TIn>::bits, Fill<TIn>::bits};
      u32x4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
        v[u] = i + u * WG < nvec ? load16<NTL>(rv + i + u * WG) : fill;
      float x[UNROLL * VE];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) Vec<TIn>::unpack(v[u], x + u * VE);
      stat_tile<UNROLL * VE, NEED_T>(st, x, c);
    }
    const int j = nvec * VE + tid;
    if (j < V) {
      const float x = load_elem(row + j);
      stat_tile<1, NEED_T>(st, &x, c);
    }
  } else {
    constexpr int K = 4 * UNROLL;
    int j = tid;
    for (; j + (K - 1) * WG < V; j += K * WG) {
      float x[K];
#pragma unroll
      for (int k = 0; k < K; ++k) x[k] = load_elem(row + j + k * WG);
      stat_tile<K, NEED_T>(st, x, c);
    }
    for (; j < V; j += WG) {
      const float x = load_elem(row + j);
      stat_tile<1, NEED_T>(st, &x, c);
    }
  }
  return st;
}

// The per-row outputs of the forward from the merged statistics st and the
// target logit zy (ignored when !valid: the row's logp is then NaN and the
// error counted).
template <bool NEED_T>
__device__ __forceinline__ void fwd_token_epilogue(const FwdArgs& a, int64_t r, const Stat& st,
                                                   float zy_in, bool valid) {
  const float logS = logf(st.s);
  const float H = NEED_T ? logS - kLn2 * st.t / st.s : 0.0f;
  const float zy = valid ? zy_in : __builtin_nanf("");
  if (!valid && a.err_count != nullptr) atomicAdd(a.err_count, 1);
  const float lse = st.m / a.T + logS;
  const float logp = (zy - st.m) / a.T - logS;
  if (a.mode == FWD_LSM) {
    a.logp[r] = logp;
    if (a.lse != nullptr) a.lse[r] = lse;
    return;
  }
  // GRPO per-token epilogue
  a.logp[r] = logp;
  a.lse[r] = lse;
  if (a.entropy != nullptr) a.entropy[r] = H;
  if (a.gathered != nullptr) a.gathered[r] = zy;
  float kl = 0.0f;
  if (a.ref_logp != nullptr) {
    const float d = a.ref_logp[r] - logp;
    kl = expm1f(d) - d;
  }
  if (a.kl != nullptr) a.kl[r] = kl;
  const float kl_term = a.beta != 0.0f ? a.beta * kl : 0.0f;
  if (a.level == GRPO_TOKEN) {
    const Ppo q = ppo_terms(logp - a.old_logp[r], a.adv[r / a.L], a.lo, a.hi);
    a.loss[r] = q.pg + kl_term;
    if (a.is_clipped != nullptr) a.is_clipped[r] = q.clipped ? 1 : 0;
  } else {
    a.loss[r] = kl_term;  // the sequence epilogue adds the sequence's pg
  }
}

template <typename TIn, int WG, int UNROLL, bool VEC, bool NEED_T, bool NTL>
__global__ __launch_bounds__(WG) void row_fwd_kernel(FwdArgs a) {
  const int64_t r = a.row0 + blockIdx.x;
  if (a.dev_rows != nullptr && r >= *a.dev_rows) return;
  const TIn* __restrict__ row = static_cast<const TIn*>(a.logits) + r * a.ld;
  const Stat st = block_reduce_stat<WG, NEED_T>(
      scan_row<TIn, WG, UNROLL, VEC, NEED_T, NTL>(row, a.V, a.c), a.c);
  if (threadIdx.x != 0) return;

  const float logS = logf(st.s);
  const float H = NEED_T ? logS - kLn2 * st.t / st.s : 0.0f;
  if (a.mode == FWD_ENTROPY) {
    a.entropy[r] = H;
    return;
  }
  const int64_t y = a.ids[r];
  const bool valid = y >= 0 && y < a.V;
  fwd_token_epilogue<NEED_T>(a, r, st, valid ? load_elem(row + y) : 0.0f, valid);
}

// Forward of the chunked loss's rows from the logits product's partial
// statistics (max and sum; no entropy): 16 rows per workgroup, four lanes of
// every wave per row, each lane merging a strided share of the row's P
// partials; the four lanes' states are merged by a fixed butterfly, the
// waves' in wave order (deterministic), and the target logit comes from zy
// (fp32).  (Sixty-four rows per workgroup left most CUs idle at a chunk's
// few thousand rows.)
constexpr int kPartialRows = 16;
template <int NW>
__global__ __launch_bounds__(64 * NW) void row_fwd_partials_kernel(FwdArgs a,
                                                                    const float* __restrict__ stat,
                                                                    int P, int64_t sl,
                                                                    const float* __restrict__ zy,
                                                                    int64_t rows) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rl = lane >> 2, sub = lane & 3;
  const int64_t r = a.row0 + int64_t(blockIdx.x) * kPartialRows + rl;
  const int64_t R = a.dev_rows != nullptr ? min(rows, int64_t(*a.dev_rows)) : rows;
  Stat st;
  stat_init(st);
  if (r < R) {
    const float* pm = stat + r;
    const float* ps = pm + int64_t(P) * sl;
#pragma unroll 4
    for (int p = 4 * w + sub; p < P; p += 4 * NW) {
      const Stat q = {pm[int64_t(p) * sl], ps[int64_t(p) * sl], 0.0f};
      st = stat_merge<false>(st, q, a.c);
    }
  }
#pragma unroll
  for (int off = 1; off < 4; off <<= 1) {
    Stat o;
    o.m = __shfl_xor(st.m, off, 64);
    o.s = __shfl_xor(st.s, off, 64);
    o.t = 0.0f;
    st = stat_merge<false>(st, o, a.c);
  }
  __shared__ Stat sh[NW][kPartialRows];
  if (sub == 0) sh[w][rl] = st;
  __syncthreads();
  if (w != 0 || sub != 0 || r >= R) return;
#pragma unroll
  for (int k = 1; k < NW; ++k) st = stat_merge<false>(st, sh[k][rl], a.c);
  const int64_t y = a.ids[r];
  const bool valid = y >= 0 && y < a.V;
  fwd_token_epilogue<false>(a, r, st, valid ? zy[r] : 0.0f, valid);
}

// sequence level: one workgroup per sequence; mask-weighted mean log-ratio,
// one clipped ratio per sequence, pg broadcast to the sequence's tokens.
__global__ __launch_bounds__(256) void seq_fwd_epilogue_kernel(SeqArgs a) {
  const int64_t b = a.b0 + blockIdx.x;
  const int64_t base = b * a.L;
  float sx = 0.0f, sm = 0.0f;
  for (int t = threadIdx.x; t < a.L; t += 256) {
    const float m = a.mask != nullptr ? float(a.mask[base + t] != 0) : 1.0f;
    sx += m * (a.logp[base + t] - a.old_logp[base + t]);
    sm += m;
  }
  __shared__ float sh[8];
  block_sum2<256>(sx, sm, sh);
  const float n = fmaxf(sm, 1.0f);
  const Ppo q = ppo_terms(sx / n, a.adv[b], a.lo, a.hi);
  if (threadIdx.x == 0) a.seq_ratio[b] = q.ratio;
  for (int t = threadIdx.x; t < a.L; t += 256) {
    a.loss[base + t] += q.pg;
    if (a.is_clipped != nullptr) a.is_clipped[base + t] = q.clipped ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
template <typename TIn, int WG>
__device__ __forceinline__ float row_dlogp(const BwdArgs& a, int64_t r) {
  if (a.mode == BWD_LSM || a.mode == BWD_ENTROPY) return a.dloss[r];
  const float logp = a.logp[r];
  const float w = a.dloss[r];
  float klg = 0.0f;
  if (a.ref_logp != nullptr && a.beta != 0.0f) klg = -a.beta * expm1f(a.ref_logp[r] - logp);
  if (a.level == GRPO_TOKEN) {
    const float A = a.adv[r / a.L];
    const Ppo q = ppo_terms(logp - a.old_logp[r], A, a.lo, a.hi);
    const float pgg = q.clipped ? 0.0f : -q.ratio * A;
    return (pgg + klg) * w;
  }
  // sequence level: per-sequence sums of dloss and of the mask
  const int64_t b = r / a.L;
  const int64_t base = b * a.L;
  float ws = 0.0f, ms = 0.0f;
  for (int t = threadIdx.x; t < a.L; t += WG) {
    ws += a.dloss[base + t];
    ms += a.mask != nullptr ? float(a.mask[base + t] != 0) : 1.0f;
  }
  __shared__ float sh[2 * (WG / 64)];
  block_sum2<WG>(ws, ms, sh);
  const float n = fmaxf(ms, 1.0f);
  const float ratio = a.seq_ratio[b];
  const float A = a.adv[b];
  const float cr = ratio < a.lo ? a.lo : (ratio > a.hi ? a.hi : ratio);
  const bool clipped = cr * A < ratio * A;
  const float coef = clipped ? 0.0f : -ratio * A;
  const float m = a.mask != nullptr ? float(a.mask[r] != 0) : 1.0f;
  return coef * ws * m / n + klg * w;
}

// store VE = Vec<TIn>::N results as one vector of the output dtype
template <typename TIn, typename TOut>
__device__ __forceinline__ void store_vec(TOut* __restrict__ out, int i, const float* x) {
  if constexpr (sizeof(TIn) == sizeof(TOut)) {
    store16(reinterpret_cast<u32x4*>(out) + i, Vec<TIn>::pack(x));
  } else {  // 4 fp32 results -> 4 bf16 (8 bytes)
    const u32x2 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(out) + i);
  }
}

// vectors [beg, end) of the row, and the elements past its last whole vector
// when `tail`; without VEC the whole row
template <typename TIn, typename TOut, int WG, bool VEC>
__device__ __forceinline__ void fill_row(TOut* __restrict__ out, int V, float value, int beg,
                                         int end, bool tail) {
  if constexpr (VEC) {
    constexpr int VE = Vec<TIn>::N;
    float x[VE];
#pragma unroll
    for (int k = 0; k < VE; ++k) x[k] = value;
    for (int i = beg + int(threadIdx.x); i < end; i += WG) store_vec<TIn, TOut>(out, i, x);
    const int j = (V / VE) * VE + threadIdx.x;
    if (tail && j < V) store_elem(out + j, value);
  } else {
    for (int j = threadIdx.x; j < V; j += WG) store_elem(out + j, value);
  }
}

// ENT: the entropy backward, dz_j = -(g/T) p_j (log p_j + H), no sampled id
template <typename TIn, typename TOut, int WG, int UNROLL, bool VEC, bool NTL, bool ENT = false>
__global__ __launch_bounds__(WG) void row_bwd_kernel(BwdArgs a) {
  // a.nchunk workgroups per row, each on WG * UNROLL consecutive vectors (the
  // last one on the rest of the row and its tail elements)
  const int64_t rl = int64_t(blockIdx.x) / a.nchunk;
  const int ch = int(int64_t(blockIdx.x) - rl * a.nchunk);
  const int64_t r = a.row0 + rl;
  const bool last = ch == a.nchunk - 1;
  if (a.dev_rows != nullptr && r >= *a.dev_rows) return;
  const float g = uniform(row_dlogp<TIn, WG>(a, r));
  const int64_t y = ENT ? 0 : a.ids[r];
  const bool valid = ENT || (y >= 0 && y < a.V);
  TOut* __restrict__ out = static_cast<TOut*>(a.dlogits) + r * a.ld_out;
  const bool zero = (g == 0.0f);
  if (threadIdx.x == 0 && ch == 0 && a.zero_row != nullptr) a.zero_row[r] = zero ? 1 : 0;
  constexpr int VEN = VEC ? Vec<TIn>::N : 1;
  const int nvec_all = a.V / VEN;
  const int vbeg = ch * (WG * UNROLL);
  const int vend = last ? nvec_all : vbeg + WG * UNROLL;
  if (!valid) {  // this workgroup's elements, one at a time
    const int e1 = last ? a.V : vend * VEN;
    for (int j = vbeg * VEN + int(threadIdx.x); j < e1; j += WG)
      store_elem(out + j, __builtin_nanf(""));
    return;
  }
  if (zero && !a.force_dense) {  // early path: no logits read, no exp
    fill_row<TIn, TOut, WG, VEC>(out, a.V, 0.0f, vbeg, vend, last);
    return;
  }
  const TIn* __restrict__ row = static_cast<const TIn*>(a.logits) + r * a.ld;
  const float coef = ENT ? -g / a.T : g / a.T;
  const float lse2 = a.lse[r] * kLog2e;
  const float c = a.c;
  const float Hr = ENT ? a.entropy[r] : 0.0f;
  const int yi = int(y);
  // one element of the dense path: u = log2 p
  auto grad_elem = [&](float x) {
    const float u = fmaf(x, c, -lse2);
    if constexpr (ENT) return coef * exp2_fast(u) * fmaf(u, kLn2, Hr);
    else return -coef * exp2_fast(u);
  };
  if constexpr (VEC) {
    constexpr int VE = Vec<TIn>::N;
    const u32x4* rv = reinterpret_cast<const u32x4*>(row);
    const int nvec = vend;
    const int vy = yi / VE, ky = yi % VE;
    int i = vbeg + int(threadIdx.x);
    for (; i + (UNROLL - 1) * WG < nvec; i += UNROLL * WG) {
      u32x4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) v[u] = load16<NTL>(rv + i + u * WG);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float x[VE];
        Vec<TIn>::unpack(v[u], x);
#pragma unroll
        for (int k = 0; k < VE; ++k) x[k] = grad_elem(x[k]);
        if (!ENT && i + u * WG == vy) {
#pragma unroll
          for (int k = 0; k < VE; ++k)
            if (k == ky) x[k] += coef;
        }
        store_vec<TIn, TOut>(out, i + u * WG, x);
      }
    }
    for (; i < nvec; i += WG) {
      float x[VE];
      Vec<TIn>::unpack(load16<NTL>(rv + i), x);
#pragma unroll
      for (int k = 0; k < VE; ++k) x[k] = grad_elem(x[k]);
      if (!ENT && i == vy) {
#pragma unroll
        for (int k = 0; k < VE; ++k)
          if (k == ky) x[k] += coef;
      }
      store_vec<TIn, TOut>(out, i, x);
    }
    const int j = nvec_all * VE + threadIdx.x;
    if (last && j < a.V) {
      float d = grad_elem(load_elem(row + j));
      if (!ENT && j == yi) d += coef;
      store_elem(out + j, d);
    }
  } else {
    for (int j = threadIdx.x; j < a.V; j += WG) {
      float d = grad_elem(load_elem(row + j));
      if (!ENT && j == yi) d += coef;
      store_elem(out + j, d);
    }
  }
}

// ---------------------------------------------------------------------------
// single pass: forward and backward of the token-level loss in one read
// ---------------------------------------------------------------------------
// When the per-token upstream weight dloss is known before the forward (a
// token-mean or sum reduction), one workgroup reads its row once into
// registers (VPT 128-bit vectors per lane), computes the row statistics,
// the per-token loss and dlogp from them, and writes dlogits from the same
// registers: the logits are read once and dlogits written once.  Vectors past
// the row end are filled with a large negative finite value, so they add
// nothing to the max or the sums and are never stored.
struct FusedArgs {
  FwdArgs f;
  void* dlogits;
  int64_t ld_out;
  const float* dloss;
  uint8_t* zero_row;
  int32_t force_dense;
};

// Opaque to the optimiser: the packed row stays the only copy in registers
// and each pass unpacks it again (two VALU ops per pair) instead of the
// compiler keeping every unpacked float alive across the passes.
__device__ __forceinline__ void keep_packed(u32x4& v) { asm volatile("" : "+v"(v)); }


template <typename TIn, int WG, int VPT, bool NEED_T>
__global__ __launch_bounds__(WG) void row_fused_kernel(FusedArgs a) {
  constexpr int VE = Vec<TIn>::N;
  const int64_t r = a.f.row0 + blockIdx.x;
  const int tid = threadIdx.x;
  const FwdArgs& f = a.f;
  const TIn* __restrict__ row = static_cast<const TIn*>(f.logits) + r * f.ld;
  const int V = f.V;
  const int nvec = V / VE;
  const float c = f.c;
  const u32x4* __restrict__ rv = reinterpret_cast<const u32x4*>(row);
  const u32x4 fill = {Fill<TIn>::bits, Fill<TIn>::bits, Fill<TIn>::bits, Fill<TIn>::bits};

  static_assert(WG >= 64 && (WG & (WG - 1)) == 0, "whole waves, a power of two of them");
  // per-row scalars first: their latency hides under the row's loads
  const int64_t y = f.ids[r];
  const float w = a.dloss[r];
  const float A = f.adv[r / f.L];
  const float old_lp = f.old_logp[r];
  const float ref_lp = f.ref_logp != nullptr ? f.ref_logp[r] : 0.0f;

  u32x4 v[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + i * WG;
    v[i] = idx < nvec ? load16<false>(rv + idx) : fill;
  }
  const int jt = nvec * VE + tid;  // the V % VE tail elements, one per lane
  const bool has_tail = jt < V;
  const float xt = has_tail ? load_elem(row + jt) : __uint_as_float(0xF149F2CAu);

  // the lane holding column y hands z_y to the others through LDS (no re-read)
  const bool valid = y >= 0 && y < V;
  const int yi = valid ? int(y) : 0;
  const int vy = yi / VE, ky = yi % VE;
  __shared__ float sh_zy;
  if (valid) {
    if (vy < nvec) {
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (tid + i * WG == vy) sh_zy = Vec<TIn>::elem(v[i], ky);
    } else if (has_tail && jt == yi) {
      sh_zy = xt;
    }
  }

  // lane statistics over the registers: max first, then the sums
  float m = xt;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    float x[VE];
    Vec<TIn>::unpack(v[i], x);
#pragma unroll
    for (int k = 0; k < VE; ++k) m = fmaxf(m, x[k]);
  }
  const float mc = m * c;
  float s = 0.0f, t = 0.0f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    keep_packed(v[i]);
    float x[VE];
    Vec<TIn>::unpack(v[i], x);
#pragma unroll
    for (int k = 0; k < VE; ++k) {
      const float d = fmaf(x[k], c, -mc);
      const float e = exp2_fast(d);
      s += e;
      if (NEED_T) t = fmaf(e, d, t);
    }
  }
  {
    const float d = fmaf(xt, c, -mc);
    const float e = exp2_fast(d);
    s += e;
    if (NEED_T) t = fmaf(e, d, t);
  }
  Stat st;
  st.m = m;
  st.s = s;
  st.t = NEED_T ? t : 0.0f;
  // A lane holding no element of the row (fewer vectors than lanes, and no
  // tail element) saw only fill values: its m is the fill and each
  // fma(x, c, -m c) above is the rounding error of m c, up to ~1e23 either
  // way, so its sums are garbage (possibly inf, and inf * 0 = NaN in the
  // merge).  It contributes the empty state instead.
  if (!(tid < nvec || has_tail)) stat_init(st);
  // Each wave merges its lanes; then wave 0 alone merges the waves' states
  // and runs the per-token epilogue, and hands the row's dlogp and lse to
  // the other waves through LDS.  (Every wave computing them alike cost a
  // sixth of the kernel's VALU instructions, the transcendental-heavy
  // epilogue fifteen times over.)
  constexpr int NW = WG / 64;
  st = wave_reduce_rescaled<NEED_T>(st, c);
  __shared__ Stat sh_st[NW];
  __shared__ float sh_g, sh_lse;
  if ((tid & 63) == 0) sh_st[tid >> 6] = st;
  __syncthreads();
  if (tid < 64) {
    st = merge_wave_states<NW, NEED_T>(sh_st, c);
    // per-token epilogue, computed alike in the lanes of wave 0
    const float logS = logf(st.s);
    const float H = NEED_T ? logS - kLn2 * st.t / st.s : 0.0f;
    const float zy = valid ? sh_zy : __builtin_nanf("");
    const float lse = st.m / f.T + logS;
    const float logp = (zy - st.m) / f.T - logS;
    float kl = 0.0f;
    if (f.ref_logp != nullptr) {
      const float d = ref_lp - logp;
      kl = expm1f(d) - d;
    }
    const Ppo q = ppo_terms(logp - old_lp, A, f.lo, f.hi);
    float klg = 0.0f;
    if (f.ref_logp != nullptr && f.beta != 0.0f) klg = -f.beta * expm1f(ref_lp - logp);
    const float g = uniform(((q.clipped ? 0.0f : -q.ratio * A) + klg) * w);
    if (tid == 0) {
      if (!valid && f.err_count != nullptr) atomicAdd(f.err_count, 1);
      f.logp[r] = logp;
      f.lse[r] = lse;
      if (f.entropy != nullptr) f.entropy[r] = H;
      if (f.kl != nullptr) f.kl[r] = kl;
      f.loss[r] = q.pg + (f.beta != 0.0f ? f.beta * kl : 0.0f);
      if (f.is_clipped != nullptr) f.is_clipped[r] = q.clipped ? 1 : 0;
      if (a.zero_row != nullptr) a.zero_row[r] = g == 0.0f ? 1 : 0;
      sh_g = g;
      sh_lse = lse;
    }
  }
  __syncthreads();
  const float g = uniform(sh_g);
  const float lse = uniform(sh_lse);
  const bool zero = (g == 0.0f);

  TIn* __restrict__ out = static_cast<TIn*>(a.dlogits) + r * a.ld_out;
  u32x4* __restrict__ ov = reinterpret_cast<u32x4*>(out);
  if (!valid) {
    for (int j = tid; j < V; j += WG) store_elem(out + j, __builtin_nanf(""));
    return;
  }
  if (zero && !a.force_dense) {
    const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * WG;
      if (idx < nvec) store16(ov + idx, z4);
    }
    if (has_tail) store_elem(out + jt, 0.0f);
    return;
  }
  const float coef = g / f.T;
  const float lse2 = lse * kLog2e;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = tid + i * WG;
    keep_packed(v[i]);
    float x[VE];
    Vec<TIn>::unpack(v[i], x);
#pragma unroll
    for (int k = 0; k < VE; ++k) x[k] = -coef * exp2_fast(fmaf(x[k], c, -lse2));
    if (idx == vy) {
#pragma unroll
      for (int k = 0; k < VE; ++k)
        if (k == ky) x[k] += coef;
    }
    if (idx < nvec) store16(ov + idx, Vec<TIn>::pack(x));
  }
  if (has_tail) {
    float d = -coef * exp2_fast(fmaf(xt, c, -lse2));
    if (jt == yi) d += coef;
    store_elem(out + jt, d);
  }
}

// ---------------------------------------------------------------------------
// launch shape dispatch
// ---------------------------------------------------------------------------
struct Shape {
  int wg, unroll;
};

// Default launch shapes (one workgroup per row), from sweeps on MI355X:
// the forward, which ends in a workgroup reduction, prefers one wave per row
// when there are few (a few thousand) short (<= 128 KB) rows, 512 x 2 for
// many short rows (on 64 KB rows 512 x 4 and 256 x 4 were within 2% either
// way, 1024 lanes 20-35% slower) and 1024 x 4 for rows past 128 KB (the
// 8192 x 151936 sequence-level forward: 0.367 ms against 0.380 at 512 x 2);
// the backward, which streams a read and a write, prefers 1024 lanes per row.
inline Shape pick_fwd_shape(int64_t rows, int64_t V, int es) {
  const LaunchOverride o = launch_override(0);
  if (o.wg > 0 && o.unroll > 0) return {o.wg, o.unroll};
  const int64_t nvec = V * es / 16;
  if (nvec <= 512) return {64, 4};
  if (rows <= 4096 && nvec <= 8192) return {64, 4};  // few, short rows
  if (nvec > 8192) return {1024, 4};                  // long rows
  return {512, 2};
}

// Backward: 256 x 2 for short rows.  Many (more than 4096) rows of up to 4096
// vectors (64 KB bf16) take four vectors per lane of 1024 lanes, all of a
// lane's loads in flight at once (on 65536 x 32000: selective backward 1.31
// ms against 1.38 at 1024 x 2, entropy backward 1.36 against 1.47); with few
// rows (2048 x 32000) 1024 x 4 measured 3% slower.  Longer rows: 1024 x 2
// when a row is one workgroup's (the fastest of 256 x 4/8, 512 x 2/4 and
// 1024 x 4 on 300 KB rows); split_rows below normally cuts them into 64 KB
// chunks of 1024 x 4 instead.
inline Shape pick_bwd_shape(int64_t rows, int64_t V, int es) {
  const LaunchOverride o = launch_override(1);
  if (o.wg > 0 && o.unroll > 0) return {o.wg, o.unroll};
  const int64_t nvec = V * es / 16;
  if (nvec <= 1024) return {256, 2};
  if (nvec <= 4096 && rows > 4096) return {1024, 4};
  return {1024, 2};
}

#define GRPO_SHAPES(X) \
  X(64, 4)             \
  X(128, 4)            \
  X(256, 2)            \
  X(256, 4)            \
  X(256, 8)            \
  X(512, 2)            \
  X(512, 4)            \
  X(1024, 2)           \
  X(1024, 4)

inline void set_row0(FwdArgs& a, int64_t r0) { a.row0 = r0; }
inline void set_row0(BwdArgs& a, int64_t r0) { a.row0 = r0; }
inline void set_row0(FusedArgs& a, int64_t r0) { a.f.row0 = r0; }

// Launch kernel k over `rows` rows, `per` workgroups of `threads` lanes
// each per row, in as many launches as one dispatch's 32-bit work-item count
// requires (each launch told its first row).
template <typename Args>
hipError_t launch_row_slices(void (*k)(Args), Args a, int64_t rows, int64_t per, int threads,
                             hipStream_t s) {
  const int64_t step = groups_per_launch(threads) / per;
  if (step < 1) return hipErrorInvalidConfiguration;
  for (int64_t r0 = 0; r0 < rows; r0 += step) {
    set_row0(a, r0);
    const int64_t n = rows - r0 < step ? rows - r0 : step;
    hipLaunchKernelGGL(k, dim3(unsigned(n * per)), dim3(threads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TIn, bool VEC, bool NEED_T, bool NTL>
hipError_t launch_fwd_t(const FwdArgs& a, int64_t rows, Shape sh, hipStream_t s) {
  if constexpr (!VEC) {
    return launch_row_slices(row_fwd_kernel<TIn, 256, 4, false, NEED_T, false>, a, rows, 1, 256,
                             s);
  } else {
#define X(W, U)                                                                          \
  if (sh.wg == W && sh.unroll == U)                                                       \
    return launch_row_slices(row_fwd_kernel<TIn, W, U, true, NEED_T, NTL>, a, rows, 1, W, s);
    GRPO_SHAPES(X)
#undef X
    return hipErrorInvalidConfiguration;
  }
}

template <typename TIn, typename TOut, bool VEC>
hipError_t launch_bwd_t(const BwdArgs& a, int64_t rows, Shape sh, bool ntl, hipStream_t s) {
  if constexpr (!VEC) {
    return launch_row_slices(row_bwd_kernel<TIn, TOut, 256, 4, false, false>, a, rows, a.nchunk,
                             256, s);
  } else {
#define X(W, U)                                                                          \
  if (sh.wg == W && sh.unroll == U)                                                       \
    return ntl ? launch_row_slices(row_bwd_kernel<TIn, TOut, W, U, true, true>, a, rows,  \
                                   a.nchunk, W, s)                                        \
               : launch_row_slices(row_bwd_kernel<TIn, TOut, W, U, true, false>, a, rows, \
                                   a.nchunk, W, s);
    GRPO_SHAPES(X)
#undef X
    return hipErrorInvalidConfiguration;
  }
}
#undef GRPO_SHAPES

inline bool rows_vec_ok(const void* p, int64_t ld, int es) {
  return aligned(p, 16) && ((ld * es) % 16) == 0;
}

template <typename TIn>
hipError_t launch_fwd_dt(const FwdArgs& a, int64_t rows, Shape sh, bool vec, bool need_t,
                         bool ntl, hipStream_t s) {
  if (!vec) return need_t ? launch_fwd_t<TIn, false, true, false>(a, rows, sh, s)
                          : launch_fwd_t<TIn, false, false, false>(a, rows, sh, s);
  if (need_t) return ntl ? launch_fwd_t<TIn, true, true, true>(a, rows, sh, s)
                         : launch_fwd_t<TIn, true, true, false>(a, rows, sh, s);
  return ntl ? launch_fwd_t<TIn, true, false, true>(a, rows, sh, s)
             : launch_fwd_t<TIn, true, false, false>(a, rows, sh, s);
}

// Logits matrices larger than this are read with non-temporal loads by the
// forward-type kernels and by the fp32 -> bf16 backward of the fused path:
// they cannot stay in the 256 MB last-level cache between the passes
// anyway, and streaming them past it measured faster (forward +8-12%, the
// fp32 backward a few percent; the same-dtype backward measured 3-5%
// slower with them and keeps normal loads).  Smaller matrices keep normal
// loads, so the backward re-reads the forward's rows from that cache.
constexpr int64_t kNtLoadBytes = int64_t(192) << 20;

int launch_fwd(const FwdArgs& a, int dtype, int64_t rows, bool need_t, hipStream_t s) {
  const int es = elem_size(dtype);
  const Shape sh = pick_fwd_shape(rows, a.V, es);
  const bool vec = rows_vec_ok(a.logits, a.ld, es);
  const bool ntl = rows * a.ld * es > kNtLoadBytes;
  const hipError_t e = dtype == GRPO_BF16
                           ? launch_fwd_dt<uint16_t>(a, rows, sh, vec, need_t, ntl, s)
                           : launch_fwd_dt<float>(a, rows, sh, vec, need_t, ntl, s);
  return e == hipSuccess ? GRPO_OK : GRPO_ERR_LAUNCH;
}

int launch_fwd_partials(const FwdArgs& a, const float* stat, int P, int64_t stat_ld,
                        const float* zy, int64_t rows, hipStream_t s) {
  if (rows <= 0) return GRPO_OK;
  constexpr int NW = 16;
  const int64_t step = groups_per_launch(64 * NW) * kPartialRows;
  FwdArgs b = a;
  for (int64_t r0 = 0; r0 < rows; r0 += step) {
    b.row0 = r0;
    const int64_t n = rows - r0 < step ? rows - r0 : step;
    hipLaunchKernelGGL((row_fwd_partials_kernel<NW>),
                       dim3(unsigned((n + kPartialRows - 1) / kPartialRows)), dim3(64 * NW), 0, s,
                       b, stat, P, stat_ld, zy, rows);
    if (hipGetLastError() != hipSuccess) return GRPO_ERR_LAUNCH;
  }
  return GRPO_OK;
}

// Rows are split into chunks, one workgroup each, that issue all of their
// loads at once and exit; each chunk recomputes its row's dlogp.  Where that
// is a few per-row scalars (token level, selective log-softmax) the chunks
// are 512 vectors (256 lanes x 2): the headline's two-pass backward 23.7
// against 26.3 us, the selective backward on 65536 x 32000 1.27 against 1.31
// ms.  At the sequence level dlogp needs the sequence's sums of dloss and
// the mask (L loads and a workgroup reduction per chunk), and the entropy
// backward does more arithmetic per element: there rows past 4096 vectors
// take 4096-vector chunks (1024 x 4; 512-vector ones made the sequence-level
// backward 0.70 against 0.54 ms and the entropy backward 11% slower).  The
// whole row per workgroup, 1024 x 2, streamed 300 KB rows at 5.1 TB/s
// against 6.35 for the same bytes as 64 KB rows.  Without 16-byte rows, or
// under a launch override, one workgroup per row.
inline void split_rows(BwdArgs& a, Shape& sh, int64_t rows, int es, bool vec) {
  a.nchunk = 1;
  if (!vec || launch_override(1).wg > 0) return;
  const bool costly = a.mode == BWD_ENTROPY || (a.mode == BWD_GRPO && a.level == GRPO_SEQUENCE);
  const Shape c = costly ? Shape{1024, 4} : Shape{256, 2};
  const int64_t cv = int64_t(c.wg) * c.unroll;
  const int64_t nvec = int64_t(a.V) * es / 16;
  if (nvec <= cv) return;
  const int64_t n = (nvec + cv - 1) / cv;
  sh = c;
  a.nchunk = int(n);
}

int launch_bwd(const BwdArgs& a0, int dtype, int64_t rows, hipStream_t s) {
  const int es = elem_size(dtype);
  Shape sh = pick_bwd_shape(rows, a0.V, es);
  const bool vec = rows_vec_ok(a0.logits, a0.ld, es) && rows_vec_ok(a0.dlogits, a0.ld_out, es);
  BwdArgs a = a0;
  split_rows(a, sh, rows, es, vec);
  const bool ntl = false;  // same-dtype backward: normal loads measured faster
  hipError_t e;
  if (dtype == GRPO_BF16) e = vec ? launch_bwd_t<uint16_t, uint16_t, true>(a, rows, sh, ntl, s)
                                  : launch_bwd_t<uint16_t, uint16_t, false>(a, rows, sh, ntl, s);
  else e = vec ? launch_bwd_t<float, float, true>(a, rows, sh, ntl, s)
               : launch_bwd_t<float, float, false>(a, rows, sh, ntl, s);
  return e == hipSuccess ? GRPO_OK : GRPO_ERR_LAUNCH;
}

// Single-pass launch: the row held in registers, 4 16-byte vectors per lane
// of one wave up to 256 vectors, 8 per lane of a 256-lane workgroup up to
// 2048, 4 per lane of a 1024-lane one up to 4096, then 16 per lane of 512
// lanes; rows longer than 128 KB do not fit.
// Returns false (nothing launched) when the row does not fit or the rows are
// not 16-byte aligned.
template <typename TIn, bool NEED_T>
hipError_t launch_fused_t(const FusedArgs& a, int64_t rows, int wg, int vpt, hipStream_t s) {
#define X(W, P)                                                                        \
  if (wg == W && vpt == P)                                                              \
    return launch_row_slices(row_fused_kernel<TIn, W, P, NEED_T>, a, rows, 1, W, s);
  X(64, 4)
  X(256, 8)
  X(256, 16)
  X(512, 8)
  X(512, 16)
  X(1024, 4)
#undef X
  return hipErrorInvalidConfiguration;
}

bool fused_shape(int64_t V, int es, int& wg, int& vpt) {
  const LaunchOverride o = parse_launch(std::getenv("GRPO_ROWS_FUSED_LAUNCH"));
  const int64_t nvec = V * es / 16;
  if (o.wg > 0 && o.unroll > 0) {
    wg = o.wg;
    vpt = o.unroll;
    return int64_t(wg) * vpt >= nvec;
  }
  // On 64 KB rows (4000 vectors, interleaved rounds on MI355X) 1024 x 4 ran
  // 46.5 us against 47.4 for 512 x 8, 48.8 for 256 x 16 and 51.5 for
  // 512 x 16; sixteen vectors per lane only for rows past 4096 vectors.
  // Rows of up to 256 vectors take one wave (no cross-wave merge).
  if (nvec <= 64 * 4) {
    wg = 64;
    vpt = 4;
  } else if (nvec <= 256 * 8) {
    wg = 256;
    vpt = 8;
  } else if (nvec <= 1024 * 4) {
    wg = 1024;
    vpt = 4;
  } else if (nvec <= 512 * 16) {
    wg = 512;
    vpt = 16;
  } else {
    return false;
  }
  return true;
}

int launch_fused(const FusedArgs& a, int dtype, int64_t rows, bool need_t, bool& launched,
                 hipStream_t s) {
  const int es = elem_size(dtype);
  launched = false;
  int wg = 0, vpt = 0;
  if (!fused_shape(a.f.V, es, wg, vpt)) return GRPO_OK;
  if (!rows_vec_ok(a.f.logits, a.f.ld, es) || !rows_vec_ok(a.dlogits, a.ld_out, es)) return GRPO_OK;
  hipError_t e;
  if (dtype == GRPO_BF16)
    e = need_t ? launch_fused_t<uint16_t, true>(a, rows, wg, vpt, s)
               : launch_fused_t<uint16_t, false>(a, rows, wg, vpt, s);
  else
    e = need_t ? launch_fused_t<float, true>(a, rows, wg, vpt, s)
               : launch_fused_t<float, false>(a, rows, wg, vpt, s);
  launched = (e == hipSuccess);
  return e == hipSuccess ? GRPO_OK : GRPO_ERR_LAUNCH;
}

template <typename T>
hipError_t launch_bwd_entropy_t(const BwdArgs& a, int64_t rows, bool vec, Shape sh,
                                hipStream_t s) {
  if (!vec)
    return launch_row_slices(row_bwd_kernel<T, T, 256, 4, false, false, true>, a, rows, a.nchunk,
                             256, s);
#define X(W, U)                                                                          \
  if (sh.wg == W && sh.unroll == U)                                                       \
    return launch_row_slices(row_bwd_kernel<T, T, W, U, true, false, true>, a, rows, a.nchunk, \
                             W, s);
  X(256, 2)
  X(1024, 2)
  X(1024, 4)
#undef X
  return hipErrorInvalidConfiguration;
}

// the entropy backward takes the backward's shape rule (256 x 2, 1024 x 4 or
// 1024 x 2; an override must name one of these)
int launch_bwd_entropy(const BwdArgs& a0, int dtype, int64_t rows, hipStream_t s) {
  const int es = elem_size(dtype);
  const bool vec = rows_vec_ok(a0.logits, a0.ld, es) && rows_vec_ok(a0.dlogits, a0.ld_out, es);
  Shape sh = pick_bwd_shape(rows, a0.V, es);
  BwdArgs a = a0;
  split_rows(a, sh, rows, es, vec);
  const hipError_t e = dtype == GRPO_BF16 ? launch_bwd_entropy_t<uint16_t>(a, rows, vec, sh, s)
                                          : launch_bwd_entropy_t<float>(a, rows, vec, sh, s);
  return e == hipSuccess ? GRPO_OK : GRPO_ERR_LAUNCH;
}

}  // namespace grpo

using namespace grpo;

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
namespace {

int check_grpo_common(const void* logits, int dtype, int64_t B, int64_t L, int64_t V, int64_t ld,
                      const int64_t* ids, const float* old_logp, const float* ref_logp,
                      const float* adv, const uint8_t* mask, const grpo_params* p) {
  if (B < 0 || L < 0 || (B > 0 && L == 0) || L > kMaxRows || (L > 0 && B > kMaxRows / L))
    return GRPO_ERR_SHAPE;
  int st = check_matrix(logits, dtype, B * L, V, ld);
  if (st != GRPO_OK) return st;
  st = check_params(p);
  if (st != GRPO_OK) return st;
  if (B * L > 0 && (ids == nullptr || old_logp == nullptr || adv == nullptr)) return GRPO_ERR_NULL;
  if (!aligned(ids, 8) || !aligned(old_logp, 4) || !aligned(ref_logp, 4) || !aligned(adv, 4))
    return GRPO_ERR_ALIGN;
  (void)mask;
  return GRPO_OK;
}

void fill_loss_params(const grpo_params* p, float& T, float& c, float& lo, float& hi) {
  T = p->temperature;
  c = kLog2e / T;
  lo = 1.0f - p->eps_low;
  hi = 1.0f + p->eps_high;
}

}  // namespace

extern "C" int grpo_logits_fwd(const void* logits, int dtype, int64_t B, int64_t L, int64_t V,
                               int64_t ld, const int64_t* ids, const float* old_logp,
                               const float* ref_logp, const float* adv, const uint8_t* mask,
                               const grpo_params* p, float* loss, float* logp, float* lse,
                               float* entropy, float* kl, uint8_t* is_clipped, float* gathered,
                               float* seq_ratio, int32_t* err_count, void* stream) {
  int st = check_grpo_common(logits, dtype, B, L, V, ld, ids, old_logp, ref_logp, adv, mask, p);
  if (st != GRPO_OK) return st;
  const int64_t rows = B * L;
  if (rows > 0 && (loss == nullptr || logp == nullptr || lse == nullptr)) return GRPO_ERR_NULL;
  if (rows > 0 && p->level == GRPO_SEQUENCE && seq_ratio == nullptr) return GRPO_ERR_NULL;
  for (const void* q : {(const void*)loss, (const void*)logp, (const void*)lse,
                        (const void*)entropy, (const void*)kl, (const void*)gathered,
                        (const void*)seq_ratio, (const void*)err_count})
    if (!aligned(q, 4)) return GRPO_ERR_ALIGN;
  if (rows == 0) return GRPO_OK;
  FwdArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.V = int32_t(V);
  a.L = int32_t(L);
  a.ids = ids;
  a.old_logp = old_logp;
  a.ref_logp = ref_logp;
  a.adv = adv;
  fill_loss_params(p, a.T, a.c, a.lo, a.hi);
  a.beta = p->beta;
  a.mode = FWD_GRPO;
  a.level = p->level;
  a.loss = loss;
  a.logp = logp;
  a.lse = lse;
  a.entropy = entropy;
  a.kl = kl;
  a.is_clipped = is_clipped;
  a.gathered = gathered;
  a.err_count = err_count;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_fwd(a, dtype, rows, entropy != nullptr, s);
  if (st != GRPO_OK || p->level != GRPO_SEQUENCE) return st;
  SeqArgs q{};
  q.L = int32_t(L);
  q.logp = logp;
  q.old_logp = old_logp;
  q.mask = mask;
  q.adv = adv;
  q.lo = a.lo;
  q.hi = a.hi;
  q.loss = loss;
  q.is_clipped = is_clipped;
  q.seq_ratio = seq_ratio;
  const int64_t step = groups_per_launch(256);
  for (int64_t b0 = 0; b0 < B; b0 += step) {
    q.b0 = b0;
    hipLaunchKernelGGL(seq_fwd_epilogue_kernel, dim3(unsigned(B - b0 < step ? B - b0 : step)),
                       dim3(256), 0, s, q);
    if (hipGetLastError() != hipSuccess) return GRPO_ERR_LAUNCH;
  }
  return GRPO_OK;
}

extern "C" int grpo_logits_bwd(const void* logits, int dtype, int64_t B, int64_t L, int64_t V,
                               int64_t ld, const int64_t* ids, const float* old_logp,
                               const float* ref_logp, const float* adv, const uint8_t* mask,
                               const grpo_params* p, const float* logp, const float* lse,
                               const float* seq_ratio, const float* dloss, void* dlogits,
                               int64_t ld_out, uint8_t* zero_row, void* stream) {
  int st = check_grpo_common(logits, dtype, B, L, V, ld, ids, old_logp, ref_logp, adv, mask, p);
  if (st != GRPO_OK) return st;
  const int64_t rows = B * L;
  if (ld_out < V) return GRPO_ERR_STRIDE;
  if (dlogits == logits && ld_out != ld) return GRPO_ERR_STRIDE;
  if (rows > 0 && (logp == nullptr || lse == nullptr || dloss == nullptr || dlogits == nullptr))
    return GRPO_ERR_NULL;
  if (rows > 0 && p->level == GRPO_SEQUENCE && seq_ratio == nullptr) return GRPO_ERR_NULL;
  if (!aligned(logp, 4) || !aligned(lse, 4) || !aligned(dloss, 4) || !aligned(seq_ratio, 4) ||
      !aligned(dlogits, elem_size(dtype)))
    return GRPO_ERR_ALIGN;
  if (rows == 0) return GRPO_OK;
  BwdArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.dlogits = dlogits;
  a.ld_out = ld_out;
  a.V = int32_t(V);
  a.L = int32_t(L);
  a.ids = ids;
  a.old_logp = old_logp;
  a.ref_logp = ref_logp;
  a.adv = adv;
  a.mask = mask;
  a.logp = logp;
  a.lse = lse;
  a.seq_ratio = seq_ratio;
  a.dloss = dloss;
  fill_loss_params(p, a.T, a.c, a.lo, a.hi);
  a.beta = p->beta;
  a.mode = BWD_GRPO;
  a.level = p->level;
  a.force_dense = (p->flags & GRPO_FLAG_FORCE_DENSE) ? 1 : 0;
  a.zero_row = zero_row;
  return launch_bwd(a, dtype, rows, static_cast<hipStream_t>(stream));
}

extern "C" int grpo_logits_fwd_bwd(const void* logits, int dtype, int64_t B, int64_t L,
                                   int64_t V, int64_t ld, const int64_t* ids,
                                   const float* old_logp, const float* ref_logp,
                                   const float* adv, const uint8_t* mask, const grpo_params* p,
                                   const float* dloss, float* loss, float* logp, float* lse,
                                   float* entropy, float* kl, uint8_t* is_clipped,
                                   void* dlogits, int64_t ld_out, uint8_t* zero_row,
                                   int32_t* err_count, void* stream) {
  int st = check_grpo_common(logits, dtype, B, L, V, ld, ids, old_logp, ref_logp, adv, mask, p);
  if (st != GRPO_OK) return st;
  if (p->level != GRPO_TOKEN) return GRPO_ERR_PARAM;
  const int64_t rows = B * L;
  if (ld_out < V) return GRPO_ERR_STRIDE;
  if (dlogits == logits && ld_out != ld) return GRPO_ERR_STRIDE;
  if (rows > 0 && (dloss == nullptr || loss == nullptr || logp == nullptr || lse == nullptr ||
                   dlogits == nullptr))
    return GRPO_ERR_NULL;
  for (const void* q : {(const void*)dloss, (const void*)loss, (const void*)logp,
                        (const void*)lse, (const void*)entropy, (const void*)kl,
                        (const void*)err_count})
    if (!aligned(q, 4)) return GRPO_ERR_ALIGN;
  if (!aligned(dlogits, elem_size(dtype))) return GRPO_ERR_ALIGN;
  if (rows == 0) return GRPO_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  FusedArgs a{};
  a.f.logits = logits;
  a.f.ld = ld;
  a.f.V = int32_t(V);
  a.f.L = int32_t(L);
  a.f.ids = ids;
  a.f.old_logp = old_logp;
  a.f.ref_logp = ref_logp;
  a.f.adv = adv;
  fill_loss_params(p, a.f.T, a.f.c, a.f.lo, a.f.hi);
  a.f.beta = p->beta;
  a.f.mode = FWD_GRPO;
  a.f.level = GRPO_TOKEN;
  a.f.loss = loss;
  a.f.logp = logp;
  a.f.lse = lse;
  a.f.entropy = entropy;
  a.f.kl = kl;
  a.f.is_clipped = is_clipped;
  a.f.err_count = err_count;
  a.dlogits = dlogits;
  a.ld_out = ld_out;
  a.dloss = dloss;
  a.zero_row = zero_row;
  a.force_dense = (p->flags & GRPO_FLAG_FORCE_DENSE) ? 1 : 0;
  bool launched = false;
  st = launch_fused(a, dtype, rows, entropy != nullptr, launched, s);
  if (st != GRPO_OK || launched) return st;
  // rows too long for registers (or not 16-byte aligned): forward then backward
  if (dlogits == logits) return GRPO_ERR_STRIDE;  // the backward would read overwritten rows
  st = launch_fwd(a.f, dtype, rows, entropy != nullptr, s);
  if (st != GRPO_OK) return st;
  BwdArgs b{};
  b.logits = logits;
  b.ld = ld;
  b.dlogits = dlogits;
  b.ld_out = ld_out;
  b.V = int32_t(V);
  b.L = int32_t(L);
  b.ids = ids;
  b.old_logp = old_logp;
  b.ref_logp = ref_logp;
  b.adv = adv;
  b.mask = mask;
  b.logp = logp;
  b.lse = lse;
  b.dloss = dloss;
  b.T = a.f.T;
  b.c = a.f.c;
  b.beta = a.f.beta;
  b.lo = a.f.lo;
  b.hi = a.f.hi;
  b.mode = BWD_GRPO;
  b.level = GRPO_TOKEN;
  b.force_dense = a.force_dense;
  b.zero_row = zero_row;
  return launch_bwd(b, dtype, rows, s);
}

extern "C" int entropy_from_logits(const void* logits, int dtype, int64_t rows, int64_t V,
                                   int64_t ld, float temperature, float* entropy,
                                   void* stream) {
  int st = check_matrix(logits, dtype, rows, V, ld);
  if (st != GRPO_OK) return st;
  if (check_temperature(temperature) != GRPO_OK) return GRPO_ERR_PARAM;
  if (rows > 0 && entropy == nullptr) return GRPO_ERR_NULL;
  if (!aligned(entropy, 4)) return GRPO_ERR_ALIGN;
  if (rows == 0) return GRPO_OK;
  FwdArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.V = int32_t(V);
  a.L = 1;
  a.T = temperature;
  a.c = kLog2e / temperature;
  a.mode = FWD_ENTROPY;
  a.entropy = entropy;
  return launch_fwd(a, dtype, rows, true, static_cast<hipStream_t>(stream));
}

extern "C" int selective_log_softmax(const void* logits, int dtype, int64_t rows, int64_t V,
                                     int64_t ld, const int64_t* ids, float temperature,
                                     float* logp, float* lse, void* stream) {
  int st = check_matrix(logits, dtype, rows, V, ld);
  if (st != GRPO_OK) return st;
  if (check_temperature(temperature) != GRPO_OK) return GRPO_ERR_PARAM;
  if (rows > 0 && (ids == nullptr || logp == nullptr)) return GRPO_ERR_NULL;
  if (!aligned(ids, 8) || !aligned(logp, 4) || !aligned(lse, 4)) return GRPO_ERR_ALIGN;
  if (rows == 0) return GRPO_OK;
  FwdArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.V = int32_t(V);
  a.L = 1;
  a.ids = ids;
  a.T = temperature;
  a.c = kLog2e / temperature;
  a.mode = FWD_LSM;
  a.logp = logp;
  a.lse = lse;
  return launch_fwd(a, dtype, rows, false, static_cast<hipStream_t>(stream));
}

extern "C" int entropy_from_logits_bwd(const void* logits, int dtype, int64_t rows, int64_t V,
                                       int64_t ld, float temperature, const float* lse,
                                       const float* entropy, const float* grad_entropy,
                                       void* dlogits, int64_t ld_out, void* stream) {
  int st = check_matrix(logits, dtype, rows, V, ld);
  if (st != GRPO_OK) return st;
  if (check_temperature(temperature) != GRPO_OK) return GRPO_ERR_PARAM;
  if (ld_out < V) return GRPO_ERR_STRIDE;
  if (dlogits == logits && ld_out != ld) return GRPO_ERR_STRIDE;
  if (rows > 0 &&
      (lse == nullptr || entropy == nullptr || grad_entropy == nullptr || dlogits == nullptr))
    return GRPO_ERR_NULL;
  if (!aligned(lse, 4) || !aligned(entropy, 4) || !aligned(grad_entropy, 4) ||
      !aligned(dlogits, elem_size(dtype)))
    return GRPO_ERR_ALIGN;
  if (rows == 0) return GRPO_OK;
  BwdArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.dlogits = dlogits;
  a.ld_out = ld_out;
  a.V = int32_t(V);
  a.L = 1;
  a.lse = lse;
  a.entropy = entropy;
  a.dloss = grad_entropy;
  a.T = temperature;
  a.c = kLog2e / temperature;
  a.mode = BWD_ENTROPY;
  return launch_bwd_entropy(a, dtype, rows, static_cast<hipStream_t>(stream));
}

extern "C" int selective_log_softmax_bwd(const void* logits, int dtype, int64_t rows, int64_t V,
                                         int64_t ld, const int64_t* ids, float temperature,
                                         const float* lse, const float* grad_logp,
                                         void* dlogits, int64_t ld_out, void* stream) {
  int st = check_matrix(logits, dtype, rows, V, ld);
  if (st != GRPO_OK) return st;
  if (check_temperature(temperature) != GRPO_OK) return GRPO_ERR_PARAM;
  if (ld_out < V) return GRPO_ERR_STRIDE;
  if (dlogits == logits && ld_out != ld) return GRPO_ERR_STRIDE;
  if (rows > 0 && (ids == nullptr || lse == nullptr || grad_logp == nullptr || dlogits == nullptr))
    return GRPO_ERR_NULL;
  if (!aligned(ids, 8) || !aligned(lse, 4) || !aligned(grad_logp, 4) ||
      !aligned(dlogits, elem_size(dtype)))
    return GRPO_ERR_ALIGN;
  if (rows == 0) return GRPO_OK;
  BwdArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.dlogits = dlogits;
  a.ld_out = ld_out;
  a.V = int32_t(V);
  a.L = 1;
  a.ids = ids;
  a.lse = lse;
  a.dloss = grad_logp;
  a.T = temperature;
  a.c = kLog2e / temperature;
  a.mode = BWD_LSM;
  return launch_bwd(a, dtype, rows, static_cast<hipStream_t>(stream));
}

extern "C" const char* grpo_status_string(int status) {
  switch (status) {
    case GRPO_OK: return "ok";
    case GRPO_ERR_NULL: return "a required pointer is NULL";
    case GRPO_ERR_SHAPE: return "a size is out of range";
    case GRPO_ERR_STRIDE: return "row stride smaller than V, or in-place with a different stride";
    case GRPO_ERR_DTYPE: return "unknown dtype";
    case GRPO_ERR_ALIGN: return "pointer not aligned to its element size";
    case GRPO_ERR_WORKSPACE: return "workspace NULL or too small";
    case GRPO_ERR_LAUNCH: return "kernel launch failed";
    case GRPO_ERR_PARAM: return "invalid loss parameter";
    case GRPO_ERR_SCRATCH:
      return "chunk needs more workspace than the no-alloc entry point's 384 MiB scratch";
    default: return "unknown status";
  }
}
