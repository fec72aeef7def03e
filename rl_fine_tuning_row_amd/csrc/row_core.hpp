// row_core.hpp -- device building blocks of the row kernels (gfx950, wave64).
//
// One workgroup owns one row of V logits.  Each lane streams 128-bit vectors
// (8 bf16 or 4 fp32) of the row, keeps a running softmax state in registers
// and the workgroup merges the per-lane states once at the end:
//
//   m = running max of the raw logits z
//   s = sum_j 2^{(z_j - m) c}                 c = log2(e) / T
//   t = sum_j 2^{(z_j - m) c} (z_j - m) c     (only when the entropy is needed)
//
// so that, with u = z / T and M = m / T,
//   lse = M + ln s,  logp_y = (z_y - m) / T - ln s,  H = ln s - ln(2) t / s.
// This is the single-read online normaliser (Milakov & Gimelshein, "Online
// normalizer calculation for softmax", 2018) extended with the entropy sum;
// the max is refreshed once per register tile, not per element.
//
// Each exponent is one FMA, fl(z c - fl(m c)): it is taken against the
// rounded product fl(m c), not against m c itself, so while a lane streams
// its sums hold every term scaled by 2^delta, delta = m c - fl(m c) (up to
// half an ulp of m c: 7.6e-6 at |m c| ~ 144, i.e. T = 0.05 on logits of a few
// units).  A max refresh rescales by 2^(fl(m_old c) - fl(m_new c)), which
// keeps that single offset; stat_exact then removes it (delta is exact as
// fma(m, c, -fl(m c))) before states of different lanes are merged, since
// lse = m / T + ln s would otherwise carry delta ln 2 -- an absolute error
// that the log-probability of a likely token (close to 0) cannot absorb.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grpo {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// initial running max: finite, so that empty lanes merge without inf - inf
constexpr float kNegBig = -1e30f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming loads and stores.  NT selects the non-temporal form (the data is
// not kept in the caches for reuse).  dlogits is written once and consumed by
// another kernel, so its stores are non-temporal; logits loads are
// non-temporal only when the host knows nothing re-reads them soon.
template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
__device__ __forceinline__ void store16(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// element loads of either input dtype (uint16_t = bf16 bits)
__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) {
  return __uint_as_float(((uint32_t)*p) << 16);
}
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = to_bf16(v); }

// 128-bit vector of the input dtype
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const u32x4& v, float* x) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
  __device__ __forceinline__ static u32x4 pack(const float* x) {
    u32x4 v;
    v.x = pack_bf16x2(x[0], x[1]);
    v.y = pack_bf16x2(x[2], x[3]);
    v.z = pack_bf16x2(x[4], x[5]);
    v.w = pack_bf16x2(x[6], x[7]);
    return v;
  }
  // element k (0..7, any lane-varying value) of the vector
  __device__ __forceinline__ static float elem(const u32x4& v, int k) {
    const uint32_t w = (k & 4) ? ((k & 2) ? v.w : v.z) : ((k & 2) ? v.y : v.x);
    return (k & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const u32x4& v, float* x) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static u32x4 pack(const float* x) {
    u32x4 v;
    v.x = __float_as_uint(x[0]); v.y = __float_as_uint(x[1]);
    v.z = __float_as_uint(x[2]); v.w = __float_as_uint(x[3]);
    return v;
  }
  // element k (0..3, any lane-varying value) of the vector
  __device__ __forceinline__ static float elem(const u32x4& v, int k) {
    return __uint_as_float((k & 2) ? ((k & 1) ? v.w : v.z) : ((k & 1) ? v.y : v.x));
  }
};

struct Stat {
  float m, s, t;
};

__device__ __forceinline__ void stat_init(Stat& st) {
  st.m = kNegBig;
  st.s = 0.0f;
  st.t = 0.0f;
}

// fold a register tile of K logits into the running state
template <int K, bool NEED_T>
__device__ __forceinline__ void stat_tile(Stat& st, const float* x, float c) {
  // The rescale must subtract the two ROUNDED products fl(m_old c) and
  // fl(m_new c) -- the references the old and the new exponents were taken
  // against.  Contracted into fma(m_old, c, -fl(m_new c)) (what HIP's default
  // -ffp-contract=fast does to `a * c - b`) it would add m_old's offset
  // delta to the old sums at every refresh, up to 1e-4 in log s over a row
  // at T = 0.05.
#pragma clang fp contract(off)
  float tm = x[0];
#pragma unroll
  for (int k = 1; k < K; ++k) tm = fmaxf(tm, x[k]);
  const float mn = fmaxf(st.m, tm);
  const float mc = mn * c;
  const float dl = st.m * c - mc;  // <= 0: rescale of the old sums (same offset)
  const float f = exp2_fast(dl);
  const float t_old = NEED_T ? f * fmaf(dl, st.s, st.t) : 0.0f;
  const float s_old = st.s;
  st.m = mn;
  float s0 = 0.0f, s1 = 0.0f, t0 = 0.0f, t1 = 0.0f;
#pragma unroll
  for (int k = 0; k < K; k += 2) {
    const float d0 = fmaf(x[k], c, -mc);
    const float e0 = exp2_fast(d0);
    s0 += e0;
    if (NEED_T) t0 = fmaf(e0, d0, t0);
    if (k + 1 < K) {
      const float d1 = fmaf(x[k + 1], c, -mc);
      const float e1 = exp2_fast(d1);
      s1 += e1;
      if (NEED_T) t1 = fmaf(e1, d1, t1);
    }
  }
  st.s = fmaf(f, s_old, s0 + s1);
  if (NEED_T) st.t = t_old + (t0 + t1);
}

// Re-reference a lane's sums from fl(m c) to the exact m c: every term was
// 2^delta too large, and each t term's exponent delta too large, so
//   s <- s 2^-delta,   t <- (t - delta s) 2^-delta.
// delta is 0 for the empty state's products that overflow (|m c| >= 2^24
// leaves no meaningful fraction anyway).
template <bool NEED_T>
__device__ __forceinline__ void stat_exact(Stat& st, float c) {
  const float mc = st.m * c;
  float delta = fmaf(st.m, c, -mc);
  delta = fabsf(delta) <= 1.0f ? delta : 0.0f;
  const float f = exp2_fast(-delta);
  if (NEED_T) st.t = (st.t - delta * st.s) * f;
  st.s *= f;
}

// Merge two states whose sums are referenced to their exact m c.
template <bool NEED_T>
__device__ __forceinline__ Stat stat_merge(const Stat& a, const Stat& b, float c) {
  const float mn = fmaxf(a.m, b.m);
  const float da = (a.m - mn) * c, db = (b.m - mn) * c;
  const float fa = exp2_fast(da), fb = exp2_fast(db);
  Stat r;
  r.m = mn;
  r.s = fa * a.s + fb * b.s;
  r.t = NEED_T ? fa * fmaf(da, a.s, a.t) + fb * fmaf(db, b.s, b.t) : 0.0f;
  return r;
}

// A wave's lane states merged with one rescale per lane: the wave's max M
// first, then each lane's sums moved from its own reference fl(m c) to
// fl(M c) (one exp2, as in stat_tile), then plain sums.  Max and sum are
// commutative, so every lane ends with the same bits.  The result is
// referenced to the exact M c.  (Merging pairwise at each shuffle costs two
// exp2 per step.)
template <bool NEED_T>
__device__ __forceinline__ Stat wave_reduce_rescaled(Stat st, float c) {
#pragma clang fp contract(off)
  float M = st.m;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float dl = st.m * c - M * c;  // <= 0, the two rounded references
  const float f = exp2_fast(dl);
  Stat r;
  r.m = M;
  r.s = f * st.s;
  r.t = NEED_T ? f * fmaf(dl, st.s, st.t) : 0.0f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    r.s += __shfl_xor(r.s, off, 64);
    if (NEED_T) r.t += __shfl_xor(r.t, off, 64);
  }
  stat_exact<NEED_T>(r, c);
  return r;
}

// The cross-wave step of a workgroup's merge, in one wave: lane i takes
// wave (i mod NW)'s state from sh and an xor butterfly merges the NW states.
// The merge is not bitwise symmetric in its operands, so lanes may differ in
// the last bit; lane 0's result is broadcast.  Every wave that runs it on
// the same data holds the same bits.
template <int NW, bool NEED_T>
__device__ __forceinline__ Stat merge_wave_states(const Stat* sh, float c) {
  static_assert((NW & (NW - 1)) == 0, "workgroup of a power-of-two number of waves");
  Stat r = sh[threadIdx.x & (NW - 1)];
#pragma unroll
  for (int off = 1; off < NW; off <<= 1) {
    Stat o;
    o.m = __shfl_xor(r.m, off, 64);
    o.s = __shfl_xor(r.s, off, 64);
    o.t = NEED_T ? __shfl_xor(r.t, off, 64) : 0.0f;
    r = stat_merge<NEED_T>(r, o, c);
  }
  r.m = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r.m)));
  r.s = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r.s)));
  if (NEED_T) r.t = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r.t)));
  return r;
}

// merge the per-lane states of the workgroup for lane 0: each wave merges
// its lanes (one rescale per lane), then wave 0 alone merges the waves'
// states; the result is lane 0's and deterministic (fixed merge order).
// Other lanes get an unspecified state (callers use lane 0's only).
// `st` is a lane's streamed state (sums referenced to fl(m c)).
template <int WG, bool NEED_T>
__device__ __forceinline__ Stat block_reduce_stat(Stat st, float c) {
  st = wave_reduce_rescaled<NEED_T>(st, c);
  if constexpr (WG == 64) {
    return st;
  } else {
    constexpr int NW = WG / 64;
    __shared__ Stat sh[NW];
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = st;
    __syncthreads();
    if (w != 0) return st;
    return merge_wave_states<NW, NEED_T>(sh, c);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// deterministic workgroup sum of two floats; valid in every lane.
// `sh` must hold 2 * WG / 64 floats; callers pass distinct buffers for
// back-to-back calls.
template <int WG>
__device__ __forceinline__ void block_sum2(float& a, float& b, float* sh) {
  a = wave_sum(a);
  b = wave_sum(b);
  if constexpr (WG > 64) {
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      sh[w] = a;
      sh[WG / 64 + w] = b;
    }
    __syncthreads();
    a = sh[0];
    b = sh[WG / 64];
#pragma unroll
    for (int k = 1; k < WG / 64; ++k) {
      a += sh[k];
      b += sh[WG / 64 + k];
    }
  }
}

__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// PPO clipped-ratio terms with NaN propagation (plain comparisons, not
// fminf/fmaxf, which would drop a NaN ratio).
struct Ppo {
  float ratio, pg;
  bool clipped;
};
__device__ __forceinline__ Ppo ppo_terms(float logratio, float A, float lo, float hi) {
  Ppo r;
  r.ratio = expf(logratio);
  const float cr = r.ratio < lo ? lo : (r.ratio > hi ? hi : r.ratio);
  const float pa = r.ratio * A, ca = cr * A;
  r.clipped = ca < pa;
  r.pg = -(r.clipped ? ca : pa);
  return r;
}

}  // namespace grpo
