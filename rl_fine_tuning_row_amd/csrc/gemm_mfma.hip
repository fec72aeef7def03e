// gemm_mfma.hip -- bf16 MFMA GEMM for the chunked fused-linear loss (see
// gemm_mfma.hpp for the layouts, tiling and fragment layout).
#include <hip/hip_runtime.h>

#include <cmath>

#include "gemm_mfma.hpp"
#include "grpo_rows.h"
#include "host_common.hpp"
#include "row_core.hpp"

namespace grpo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

constexpr int NTHREADS = 256;

// Tile configuration: BM x BN block tile, BK deep K step, 4 waves in a 2 x 2
// grid, each wave (BM/2) x (BN/2) = TM x TN tiles of 32 x 32.
template <int BM_, int BN_, int BK_, int WPE_ = 1>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WPE = WPE_;  // waves per SIMD the register budget must allow
  static constexpr int LROW = BK + 8;  // LDS row pitch in bf16 (16-byte pad)
  static constexpr int TM = BM / 64, TN = BN / 64;
};

// Staging of one ROWS x BK operand tile (rows = M or N index), in registers.
//  K-contiguous: CPT = ROWS*BK/8/256 16-byte chunks per lane, chunk
//    c = lane + 256 i covers row c / (BK/8), k-offset 8 (c % (BK/8)).
//  MN-contiguous: the tile is (BK/8) x (ROWS/8) blocks of 8 x 8; TPB lanes
//    share a block, each loading KPT = 8 / TPB consecutive K-rows of it.
//    Successive blocks step along K first, so the lanes of a wave write
//    their transposed rows side by side in LDS (no bank conflicts).
template <int ROWS, int BK, bool KC>
struct Stage {
  static constexpr int CPT = ROWS * BK / 8 / NTHREADS;
  static constexpr int BLOCKS = (BK / 8) * (ROWS / 8);
  static constexpr int TPB = NTHREADS / BLOCKS;
  static constexpr int KPT = 8 / (TPB > 0 ? TPB : 1);
  static constexpr int NREG = KC ? CPT : KPT;
  static_assert(KC ? (CPT >= 1) : (TPB >= 1 && TPB <= 8 && 8 % TPB == 0), "bad tile");

  __device__ __forceinline__ static void load(const uint16_t* __restrict__ P, int64_t ld,
                                              int extent, int r0, int k0, int kend,
                                              v4u (&v)[NREG]) {
    const int t = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = t + NTHREADS * i;
        const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        const bool ok = (r0 + row < extent) && (k0 + kc < kend);
        v[i] = ok ? *reinterpret_cast<const v4u*>(P + int64_t(r0 + row) * ld + k0 + kc)
                  : v4u{0u, 0u, 0u, 0u};
      }
    } else {
      const int b = t / TPB, q = t % TPB;
      const int kb = b % (BK / 8), rb = b / (BK / 8);
      const bool col_ok = r0 + rb * 8 < extent;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int k = k0 + kb * 8 + q * KPT + i;
        const bool ok = col_ok && (k < kend);
        v[i] = ok ? *reinterpret_cast<const v4u*>(P + int64_t(k) * ld + r0 + rb * 8)
                  : v4u{0u, 0u, 0u, 0u};
      }
    }
  }

  // write to an LDS tile laid out [row][k] with pitch LROW
  template <int LROW>
  __device__ __forceinline__ static void store(uint16_t* __restrict__ lds, const v4u (&v)[NREG]) {
    const int t = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = t + NTHREADS * i;
        const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        *reinterpret_cast<v4u*>(lds + row * LROW + kc) = v[i];
      }
    } else {
      // transpose: element e of the 8 rows' values of K-row i goes to LDS
      // row (rb*8 + e), column kb*8 + q*KPT + i; pairs of K-rows share one
      // 32-bit word (one v_perm_b32 each)
      const int b = t / TPB, q = t % TPB;
      const int kb = b % (BK / 8), rb = b / (BK / 8);
      uint16_t* base = lds + (rb * 8) * LROW + kb * 8 + q * KPT;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[KPT / 2];
#pragma unroll
        for (int i = 0; i < KPT / 2; ++i) {
          const uint32_t lo = v[2 * i][e >> 1], hi = v[2 * i + 1][e >> 1];
          w[i] = __builtin_amdgcn_perm(hi, lo, sel);
        }
        uint16_t* dst = base + e * LROW;
        if constexpr (KPT == 2) {
          *reinterpret_cast<uint32_t*>(dst) = w[0];
        } else if constexpr (KPT == 4) {
          *reinterpret_cast<v2u*>(dst) = v2u{w[0], w[1]};
        } else {
          *reinterpret_cast<v4u*>(dst) = v4u{w[0], w[1], w[2], w[3]};
        }
      }
    }
  }
};

// Operand handling of the pipelined kernel, one ROWS x BK tile per K step,
// staged as NREG 16-byte chunks per lane (chunk i of lane t is chunk
// t + 256 i of the tile).
//  K-contiguous: LDS [row][k], pitch BK + 8; a fragment is one 128-bit read.
//  MN-contiguous: LDS [k][row], pitch ROWS + 32, filled by plain 16-byte
//    copies (no register transpose); a fragment is two ds_read_b64_tr_b16.
//    That instruction, within each 16-lane group, gives lane i as element j
//    the 16-bit value at (address of lane 4 j + i / 4) + i % 4 (checked on
//    MI355X).  So if lane q of the group points at K-row kb + q / 4, columns
//    c + 4 (q % 4) .. +3, lane i receives rows kb .. kb+3 of column c + i:
//    the K-run the MFMA fragment wants.  The 32-element pad puts the four
//    K-rows one read touches on disjoint bank quarters.
// load_one_clamped reads from an always-valid address and reports whether
// the chunk lies inside the operand (the caller stores zeros otherwise).
template <int ROWS, int BK, bool KC>
struct PipeOp;

template <int ROWS, int BK>
struct PipeOp<ROWS, BK, true> {
  static constexpr int PITCH = BK + 8;
  static constexpr int ELEMS = ROWS * PITCH;
  static constexpr int CPR = BK / 8;  // 16-byte chunks per row
  static constexpr int NREG = ROWS * CPR / NTHREADS;
  static constexpr int READS = 1;  // LDS instructions per fragment
  static_assert(NREG >= 1, "bad tile");
  __device__ __forceinline__ static int row_of(int i) { return (threadIdx.x + NTHREADS * i) / CPR; }
  __device__ __forceinline__ static int k_of(int i) { return ((threadIdx.x + NTHREADS * i) % CPR) * 8; }
  __device__ __forceinline__ static v4u load_one(const uint16_t* __restrict__ P, int64_t ld,
                                                 int r0, int k0, int i) {
    return *reinterpret_cast<const v4u*>(P + int64_t(r0 + row_of(i)) * ld + k0 + k_of(i));
  }
  // the same address split into a wave-uniform part (one per K step) and the
  // lane's chunk offset (the same every step)
  __device__ __forceinline__ static int64_t chunk_offset(int64_t ld, int i) {
    return int64_t(row_of(i)) * ld + k_of(i);
  }
  // the same with the row clamped to the operand's last (extent > r0): a
  // tile that overhangs M or N reads valid rows there, whose results are
  // never stored
  __device__ __forceinline__ static int64_t chunk_offset_clamped(int64_t ld, int i, int r0,
                                                                 int extent) {
    return int64_t(min(row_of(i), extent - 1 - r0)) * ld + k_of(i);
  }
  __device__ __forceinline__ static const uint16_t* step_base(const uint16_t* P, int64_t ld, int r0,
                                                              int k0) {
    return P + int64_t(r0) * ld + k0;
  }
  // requires extent >= 1 and kend >= 8
  __device__ __forceinline__ static v4u load_one_clamped(const uint16_t* __restrict__ P,
                                                         int64_t ld, int extent, int r0, int k0,
                                                         int kend, int i, bool& in) {
    const int row = r0 + row_of(i), k = k0 + k_of(i);
    in = (row < extent) && (k < kend);
    return *reinterpret_cast<const v4u*>(P + int64_t(min(row, extent - 1)) * ld + min(k, kend - 8));
  }
  __device__ __forceinline__ static void store_one(uint16_t* __restrict__ lds, int i, v4u v) {
    *reinterpret_cast<v4u*>(lds + row_of(i) * PITCH + k_of(i)) = v;
  }
  // lane's fragment base for the wave's half `h` of the tile's rows
  __device__ __forceinline__ static int lane_offset(int h, int lane) {
    return (h * (ROWS / 2) + (lane & 31)) * PITCH + 8 * (lane >> 5);
  }
  // fragment of 32-row block i, K sub-step s (16 deep)
  __device__ __forceinline__ static bf16x8 frag(const uint16_t* tile, int off, int i, int s) {
    return *reinterpret_cast<const bf16x8*>(tile + off + i * 32 * PITCH + s * 16);
  }
};

template <int ROWS, int BK>
struct PipeOp<ROWS, BK, false> {
  static constexpr int PITCH = ROWS + 32;
  static constexpr int ELEMS = BK * PITCH;
  static constexpr int RC = ROWS / 8;  // 16-byte chunks per K-row
  static constexpr int NREG = ROWS * BK / 8 / NTHREADS;
  static constexpr int READS = 2;
  static_assert(NREG >= 1, "bad tile");
  __device__ __forceinline__ static int k_of(int i) { return (threadIdx.x + NTHREADS * i) / RC; }
  __device__ __forceinline__ static int col_of(int i) { return ((threadIdx.x + NTHREADS * i) % RC) * 8; }
  __device__ __forceinline__ static v4u load_one(const uint16_t* __restrict__ P, int64_t ld,
                                                 int r0, int k0, int i) {
    return *reinterpret_cast<const v4u*>(P + int64_t(k0 + k_of(i)) * ld + r0 + col_of(i));
  }
  __device__ __forceinline__ static int64_t chunk_offset(int64_t ld, int i) {
    return int64_t(k_of(i)) * ld + col_of(i);
  }
  // columns clamped to the last 16-byte chunk of the extent (extent % 8 == 0,
  // extent > r0)
  __device__ __forceinline__ static int64_t chunk_offset_clamped(int64_t ld, int i, int r0,
                                                                 int extent) {
    return int64_t(k_of(i)) * ld + min(col_of(i), extent - 8 - r0);
  }
  __device__ __forceinline__ static const uint16_t* step_base(const uint16_t* P, int64_t ld, int r0,
                                                              int k0) {
    return P + int64_t(k0) * ld + r0;
  }
  // requires extent % 8 == 0, extent >= 8 and kend >= 1
  __device__ __forceinline__ static v4u load_one_clamped(const uint16_t* __restrict__ P,
                                                         int64_t ld, int extent, int r0, int k0,
                                                         int kend, int i, bool& in) {
    const int k = k0 + k_of(i), row = r0 + col_of(i);
    in = (row < extent) && (k < kend);
    return *reinterpret_cast<const v4u*>(P + int64_t(min(k, kend - 1)) * ld + min(row, extent - 8));
  }
  __device__ __forceinline__ static void store_one(uint16_t* __restrict__ lds, int i, v4u v) {
    *reinterpret_cast<v4u*>(lds + k_of(i) * PITCH + col_of(i)) = v;
  }
  // lane l (group G = l / 16, q = l % 16) points at K-row 8 (G / 2) + q / 4,
  // column 16 (G % 2) + 4 (q % 4) of its wave's half of the rows
  __device__ __forceinline__ static int lane_offset(int h, int lane) {
    return (8 * (lane >> 5) + ((lane & 15) >> 2)) * PITCH + h * (ROWS / 2) +
           16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  }
  __device__ __forceinline__ static bf16x8 frag(const uint16_t* tile, int off, int i, int s) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const uint16_t* p = tile + off + s * 16 * PITCH + i * 32;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * PITCH));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

template <class C, bool A_KC, bool B_KC, int MODE>
__global__ __launch_bounds__(NTHREADS, C::WPE) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, LROW = C::LROW, TM = C::TM, TN = C::TN;
  using SA = Stage<BM, BK, A_KC>;
  using SB = Stage<BN, BK, B_KC>;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LROW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LROW];

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of tiles (successive m for one n) so tiles that share
  // a B panel share that XCD's L2.
  const int tiles = g.tiles_m * g.tiles_n;
  const int id = blockIdx.x;
  const int q = tiles / 8, rr = tiles % 8;
  const int xcd = id % 8, j = id / 8;
  const int t = xcd * q + min(xcd, rr) + j;
  const int tm = t % g.tiles_m, tn = t / g.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  // extents read on the device (compacted rows): tiles past them have no work
  if (g.dev_m != nullptr) g.M = min(g.M, *g.dev_m);
  if (g.dev_k != nullptr) g.K = min(g.K, *g.dev_k);
  if (m0 >= g.M) return;

  const int z = blockIdx.y;
  const int kbeg = z * g.k_per_split;
  const int kend = min(g.K, kbeg + g.k_per_split);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < TN; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;

  v4u ra[SA::NREG], rb[SB::NREG];
  SA::load(g.A, g.lda, g.M, m0, kbeg, kend, ra);
  SB::load(g.B, g.ldb, g.N, n0, kbeg, kend, rb);
  SA::template store<LROW>(As[0], ra);
  SB::template store<LROW>(Bs[0], rb);
  __syncthreads();

  int buf = 0;
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) {
      SA::load(g.A, g.lda, g.M, m0, k0 + BK, kend, ra);
      SB::load(g.B, g.ldb, g.N, n0, k0 + BK, kend, rb);
    }
    const uint16_t* a_l = As[buf] + (wm * (BM / 2) + (lane & 31)) * LROW + 8 * (lane >> 5);
    const uint16_t* b_l = Bs[buf] + (wn * (BN / 2) + (lane & 31)) * LROW + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(a_l + i * 32 * LROW + s * 16);
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
        fb[jj] = *reinterpret_cast<const bf16x8*>(b_l + jj * 32 * LROW + s * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[jj], acc[i][jj], 0, 0, 0);
    }
    if (more) {
      SA::template store<LROW>(As[buf ^ 1], ra);
      SB::template store<LROW>(Bs[buf ^ 1], rb);
    }
    __syncthreads();
    buf ^= 1;
  }

  float* Cp = g.C + int64_t(z) * g.split_stride;
  const int nl = lane & 31, mg = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) {
      const int n = n0 + wn * (BN / 2) + jj * 32 + nl;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + mg + (r & 3);
        if (m < g.M) {
          float* p = Cp + int64_t(m) * g.ldc + n;
          if constexpr (MODE == GEMM_ACCUM) *p += acc[i][jj][r];
          else *p = acc[i][jj][r];
        }
      }
    }
  }
}

// Spread U = 0 .. NU-1 MFMAs evenly over R LDS reads, W LDS writes and V
// global loads (one MFMA, then its share of each), for sched_group_barrier.
template <int U, int NU, int R, int W, int V>
__device__ __forceinline__ void sched_mix() {
  if constexpr (U < NU) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    constexpr int r = (R * (U + 1)) / NU - (R * U) / NU;
    constexpr int w = (W * (U + 1)) / NU - (W * U) / NU;
    constexpr int v = (V * (U + 1)) / NU - (V * U) / NU;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // DS read
    if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);  // DS write
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);  // VMEM read
    sched_mix<U + 1, NU, R, W, V>();
  }
}

// K loop of the pipelined kernel; EDGE selects clamped, masked staging
// (tiles that overhang M, N or the K range) over plain loads.  A K step on
// LDS buffer b is four 16-deep sub-steps of 16 MFMAs, each fed by fragments
// read during the sub-step before:
//  sub-steps 0-2 also write a third of the next step's staged chunks into
//    buffer b^1 and, into each register just written out, load the chunk of
//    the step after next (a full step of latency cover), so that no
//    sub-step carries a burst of LDS writes or global loads;
//  a barrier then makes b^1 whole (and ends every read of b);
//  sub-step 3 reads the next step's first fragments from b^1, so nothing
//    waits on LDS after the barrier.
// The body has no branches; sched_group_barrier interleaves the memory
// instructions with the MFMAs and sched_barrier keeps the sub-steps apart.
template <class C, bool A_KC, bool B_KC, bool EDGE>
__device__ __forceinline__ void pipe_mainloop(
    const GemmArgs& g, int m0, int n0, int kbeg, int kend,
    uint16_t (*As)[PipeOp<C::BM, C::BK, A_KC>::ELEMS],
    uint16_t (*Bs)[PipeOp<C::BN, C::BK, B_KC>::ELEMS], f32x16 (&acc)[C::TM][C::TN]) {
  constexpr int BK = C::BK, TM = C::TM, TN = C::TN;
  static_assert(BK == 64, "four 16-deep sub-steps per K step");
  using OA = PipeOp<C::BM, BK, A_KC>;
  using OB = PipeOp<C::BN, BK, B_KC>;
  constexpr int NA = OA::NREG, NW = NA + OB::NREG;
  static_assert(NW <= 32, "one in-bounds bit per chunk");
  constexpr int NR = TM * OA::READS + TN * OB::READS;  // LDS reads per sub-step
  // chunks written (and reloaded) in sub-steps 0, 1, 2: [0, W1), [W1, W2), [W2, NW)
  constexpr int W1 = (NW + 2) / 3, W2 = W1 + (NW - W1 + 1) / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  v4u r[NW];
  uint32_t in_bits = ~0u;
  // interior tiles: each chunk's address is a wave-uniform base for the K
  // step (scalar arithmetic) plus the lane's fixed offset, so a load costs one
  // 64-bit add instead of a 64-bit multiply per chunk and step
  int64_t off[NW];
  if constexpr (!EDGE) {
#pragma unroll
    for (int c = 0; c < NW; ++c)
      off[c] = c < NA ? OA::chunk_offset_clamped(g.lda, c, m0, g.M)
                      : OB::chunk_offset_clamped(g.ldb, c - NA, n0, g.N);
  }
  auto load_chunk = [&](int c, int k) {
    if constexpr (EDGE) {
      bool in;
      if (c < NA) r[c] = OA::load_one_clamped(g.A, g.lda, g.M, m0, k, kend, c, in);
      else r[c] = OB::load_one_clamped(g.B, g.ldb, g.N, n0, k, kend, c - NA, in);
      in_bits = in ? (in_bits | (1u << c)) : (in_bits & ~(1u << c));
    } else {
      const uint16_t* base = c < NA ? OA::step_base(g.A, g.lda, m0, k)
                                    : OB::step_base(g.B, g.ldb, n0, k);
      r[c] = *reinterpret_cast<const v4u*>(base + off[c]);
    }
  };
  auto store_chunk = [&](int c, int b) {
    v4u v = r[c];
    if constexpr (EDGE) v = ((in_bits >> c) & 1u) ? v : v4u{0u, 0u, 0u, 0u};
    if (c < NA) OA::store_one(As[b], c, v);
    else OB::store_one(Bs[b], c - NA, v);
  };
  const int a_off = OA::lane_offset(wm, lane);
  const int b_off = OB::lane_offset(wn, lane);
  bf16x8 fa[2][TM], fb[2][TN];
  auto frags = [&](int set, int b, int s) {
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[set][i] = OA::frag(As[b], a_off, i, s);
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) fb[set][jj] = OB::frag(Bs[b], b_off, jj, s);
  };
  // operands swapped (B fragment as the row operand): see the epilogue
  auto mfmas = [&](int set) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][jj], fa[set][i],
                                                            acc[i][jj], 0, 0, 0);
  };

  // the last steps reload the final step's tile (in bounds, never used)
  const int last = ((kend - 1 - kbeg) / BK) * BK + kbeg;
#pragma unroll
  for (int c = 0; c < NW; ++c) load_chunk(c, kbeg);
#pragma unroll
  for (int c = 0; c < NW; ++c) store_chunk(c, 0);
  // the second step's loads in chunk order, after the stores: the loop then
  // finds them outstanding in the order its own loads leave them, and waits
  // for each chunk only as long as needed
  __builtin_amdgcn_sched_barrier(0);
  const int k1 = min(kbeg + BK, last);
#pragma unroll
  for (int c = 0; c < NW; ++c) load_chunk(c, k1);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  frags(0, 0, 0);

  int b = 0;
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    const int k2 = min(k0 + 2 * BK, last);
    __builtin_amdgcn_sched_barrier(0);
    frags(1, b, 1);
    mfmas(0);
#pragma unroll
    for (int c = 0; c < W1; ++c) {
      store_chunk(c, b ^ 1);
      load_chunk(c, k2);
    }
    sched_mix<0, 8, NR, 0, 0>();
    sched_mix<0, 8, 0, W1, W1>();
    __builtin_amdgcn_sched_barrier(0);
    frags(0, b, 2);
    mfmas(1);
#pragma unroll
    for (int c = W1; c < W2; ++c) {
      store_chunk(c, b ^ 1);
      load_chunk(c, k2);
    }
    sched_mix<0, 8, NR, 0, 0>();
    sched_mix<0, 8, 0, W2 - W1, W2 - W1>();
    __builtin_amdgcn_sched_barrier(0);
    frags(1, b, 3);
    mfmas(0);
#pragma unroll
    for (int c = W2; c < NW; ++c) {
      store_chunk(c, b ^ 1);
      load_chunk(c, k2);
    }
    sched_mix<0, 8, NR, 0, 0>();
    sched_mix<0, 8, 0, NW - W2, NW - W2>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    frags(0, b ^ 1, 0);
    mfmas(1);
    sched_mix<0, 8, NR, 0, 0>();
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    b ^= 1;
  }
}

// Software-pipelined kernel for the 256 x 256 x 64 tile (one wave per SIMD,
// so the wave itself must hide every latency; see pipe_mainloop).
template <class C, bool A_KC, bool B_KC, int MODE>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_pipe_kernel(GemmArgs g) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, TM = C::TM, TN = C::TN;
  static_assert(BK == 64 && TM == 4 && TN == 4, "pipelined kernel expects 256 x 256 x 64");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][PipeOp<BM, BK, A_KC>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][PipeOp<BN, BK, B_KC>::ELEMS];
  // extents read on the device (compacted rows): the grid is sized for the
  // host's bound and only the tiles inside the device extent have work
  if (g.dev_m != nullptr) g.M = min(g.M, *g.dev_m);
  if (g.dev_k != nullptr) g.K = min(g.K, *g.dev_k);
  // Workgroups are dispatched round-robin over the 8 XCDs in linear order.
  // Number the active tiles of every K-split 0 .. total-1, give each XCD an
  // equal contiguous run of them and let the rest return, so that inactive
  // tiles (rows past the device extent) leave no XCD idle.  Within a split
  // the run takes successive m for one n (tiles that share a B panel share
  // that XCD's L2) unless C has at most 8 column tiles: then successive n
  // for one m, so that the 32 tiles an XCD runs at once read 8 A panels and
  // every B panel (12 distinct panels) instead of 32 A panels and one B.
  const int tiles_m = (g.M + BM - 1) / BM;
  const int per_split = tiles_m * g.tiles_n;
  const int total = per_split * int(gridDim.y);
  const int id = int(blockIdx.x + gridDim.x * blockIdx.y);
  if (id >= total) return;
  const int q = total / 8, rr = total % 8;
  const int xcd = id % 8, j = id / 8;
  const int t = xcd * q + min(xcd, rr) + j;
  const int z = t / per_split, tt = t % per_split;
  const bool n_fast = g.tiles_n <= 8;
  const int tm = n_fast ? tt / g.tiles_n : tt % tiles_m;
  const int tn = n_fast ? tt % g.tiles_n : tt / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = z * g.k_per_split;
  const int kend = min(g.K, kbeg + g.k_per_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < TN; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;

  if (kend > kbeg) {
    // whole K steps take the unmasked loop, also in tiles that overhang M or
    // N (their loads clamped into the operands; the epilogues store no row or
    // column past C); a partial K step needs the masked one
    const bool whole_k = (kend - kbeg) % BK == 0;
    if (whole_k) pipe_mainloop<C, A_KC, B_KC, false>(g, m0, n0, kbeg, kend, As, Bs, acc);
    else pipe_mainloop<C, A_KC, B_KC, true>(g, m0, n0, kbeg, kend, As, Bs, acc);
  }

  // Epilogue.  The MFMAs ran with the operands swapped (B fragment as the
  // row operand), so accumulator r of lane l holds C[m][n] at
  // m = 32 i + l % 32, n = 32 jj + 8 (r / 4) + 4 (l / 32) + r % 4: four
  // consecutive columns per lane.  Each wave stages one 32 x 128 block of
  // its 128 x 128 tile at a time in its own LDS slice (16-byte writes), reads
  // it back as whole rows and writes C with 16-byte stores, two 512-byte
  // rows per instruction (the accumulate mode loads C the same way first).
  // Tiles inside C take a path with no per-row checks: the checked one
  // costs several thousand scalar and branch instructions per tile.
  __syncthreads();  // every wave is done with the operand tiles
  constexpr int EP = 128 + 4;  // staging pitch in floats
  static_assert(4 * 32 * EP * 4 <= int(sizeof(As)), "staging fits the A tiles");
  float* stage = reinterpret_cast<float*>(&As[0][0]) + wave * (32 * EP);
  float* const stage0 = stage;
  float* Cp = g.C + int64_t(z) * g.split_stride;
  const int mw = m0 + wm * (BM / 2), nw = n0 + wn * (BN / 2);
  const int col = 4 * (lane & 31);
  const int n = nw + col;
  auto stage_block = [&](int i) {
#pragma unroll
    for (int jj = 0; jj < TN; ++jj)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[i][jj][4 * q], acc[i][jj][4 * q + 1], acc[i][jj][4 * q + 2],
                         acc[i][jj][4 * q + 3]};
        *reinterpret_cast<f32x4*>(stage + (lane & 31) * EP + 32 * jj + 8 * q + 4 * (lane >> 5)) = v;
      }
  };
  // rows 2 u + lane / 32 of block i, columns 4 (lane % 32) .. +3
  auto staged = [&](int u) {
    return *reinterpret_cast<const f32x4*>(stage + (2 * u + (lane >> 5)) * EP + col);
  };
  // store mode streams C past the caches (the logits of a chunk, 1.8 GB,
  // would otherwise evict the operand panels the product re-reads; measured
  // 3% off a fused batch); accumulate keeps the C it just read
  auto put = [&](float* p, const f32x4& v) {
    if constexpr (MODE == GEMM_STORE) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
    else *reinterpret_cast<f32x4*>(p) = v;
  };
  if constexpr (MODE == GEMM_LOGITS) {
    // Per 32-row block: each row's 128 columns of this wave are split
    // between lanes l and l^32 (64 each, in registers).  Each lane folds its
    // 64 into an online softmax state (max and sum; the chunked loss needs no
    // entropy), the pair merges, and one partial per row and half-tile is
    // written.  The block then goes through the LDS
    // staging for the target logit of each row (fp32) and for the bf16 copy
    // (four 256-byte row pieces per instruction; non-temporal: the row pass
    // reads it only after the product's other tiles).
    const float c = g.cscale;
    const int P = 2 * g.tiles_n, p = 2 * tn + wn;
    const int64_t sl = g.stat_ld;
    float* pm = g.stat + int64_t(p) * sl;
    float* ps = pm + int64_t(P) * sl;
    float* stage = stage0;
    const int cb = 8 * (lane & 15);  // first of this lane's 8 columns in a row piece
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      stage_block(i);
      // Columns past N leave the fold.  With N % 8 == 0 that is decided per
      // 8-column group, the same for every lane (uniform), and a wave with
      // no column left keeps the empty state rather than fold the fill.
      const int nv = g.N - nw;  // columns of this wave's half inside C
      float x[4 * 16];          // x[16 jj + r] = acc[i][jj][r]
      Stat st;
      stat_init(st);
      if (nv >= BN / 2) {  // the whole half inside C: no per-element select
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) x[16 * jj + r] = acc[i][jj][r];
        stat_tile<64, false>(st, x, c);
      } else if (nv > 0) {
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            x[16 * jj + r] = 32 * jj + 8 * (r >> 2) < nv ? acc[i][jj][r] : kNegBig;
        stat_tile<64, false>(st, x, c);
      }
      stat_exact<false>(st, c);
      Stat o;
      o.m = __shfl_xor(st.m, 32, 64);
      o.s = __shfl_xor(st.s, 32, 64);
      o.t = 0.0f;
      st = stat_merge<false>(st, o, c);
      if (lane < 32) {
        const int m = mw + 32 * i + lane;
        if (m < g.M) {
          pm[m] = st.m;
          ps[m] = st.s;
          const int64_t y = g.ids[m];
          if (y >= nw && y < nw + BN / 2 && y < g.N) g.zy[m] = stage[lane * EP + int(y - nw)];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int row = 4 * u + (lane >> 4);
        const int m = mw + 32 * i + row;
        const f32x4 a = *reinterpret_cast<const f32x4*>(stage + row * EP + cb);
        const f32x4 b = *reinterpret_cast<const f32x4*>(stage + row * EP + cb + 4);
        if (m >= g.M) continue;
        uint16_t* q = g.z16 + int64_t(m) * g.ldc + nw + cb;
        if (nw + cb + 8 <= g.N) {
          const v4u w = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                         pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
          __builtin_nontemporal_store(w, reinterpret_cast<v4u*>(q));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (nw + cb + e < g.N) q[e] = to_bf16(e < 4 ? a[e] : b[e - 4]);
        }
      }
      // one row block at a time (interleaving them spills registers)
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  if (g.vec_c && m0 + BM <= g.M && n0 + BN <= g.N) {
    const int64_t pair = 2 * g.ldc;  // two rows per instruction
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      stage_block(i);
      float* p0 = Cp + int64_t(mw + 32 * i + (lane >> 5)) * g.ldc + n;
      f32x4 cur[16];
      if constexpr (MODE == GEMM_ACCUM) {
#pragma unroll
        for (int u = 0; u < 16; ++u) cur[u] = *reinterpret_cast<const f32x4*>(p0 + u * pair);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if constexpr (MODE == GEMM_ACCUM) cur[u] += staged(u);
        else cur[u] = staged(u);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) put(p0 + u * pair, cur[u]);
    }
    return;
  }
  const bool full_n = g.vec_c && (n + 3 < g.N);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    stage_block(i);
    f32x4 cur[16];
    if constexpr (MODE == GEMM_ACCUM) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int m = mw + 32 * i + 2 * u + (lane >> 5);
        float* p = Cp + int64_t(m) * g.ldc + n;
        if (m < g.M && full_n) {
          cur[u] = *reinterpret_cast<const f32x4*>(p);
        } else {
          cur[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          if (m < g.M)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < g.N) cur[u][e] = p[e];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if constexpr (MODE == GEMM_ACCUM) cur[u] += staged(u);
      else cur[u] = staged(u);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int m = mw + 32 * i + 2 * u + (lane >> 5);
      if (m >= g.M) continue;
      float* p = Cp + int64_t(m) * g.ldc + n;
      if (full_n) {
        put(p, cur[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < g.N) p[e] = cur[u][e];
      }
    }
  }
}

template <class C, bool A_KC, bool B_KC>
hipError_t launch_pipe(int mode, GemmArgs g, int splits, hipStream_t s) {
  // 16-byte accesses to C need every row start (and split slab) 16-byte aligned
  g.vec_c = (reinterpret_cast<uintptr_t>(g.C) % 16 == 0) && (g.ldc % 4 == 0) &&
            (splits == 1 || g.split_stride % 4 == 0);
  g.tiles_m = (g.M + C::BM - 1) / C::BM;
  g.tiles_n = (g.N + C::BN - 1) / C::BN;
  const dim3 grid(unsigned(g.tiles_m * g.tiles_n), unsigned(splits));
  if (mode == GEMM_ACCUM)
    hipLaunchKernelGGL((gemm_bf16_pipe_kernel<C, A_KC, B_KC, GEMM_ACCUM>), grid, dim3(NTHREADS), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_bf16_pipe_kernel<C, A_KC, B_KC, GEMM_STORE>), grid, dim3(NTHREADS), 0, s, g);
  return hipGetLastError();
}

template <class C, bool A_KC, bool B_KC>
hipError_t launch(int mode, GemmArgs g, int splits, hipStream_t s) {
  g.tiles_m = (g.M + C::BM - 1) / C::BM;
  g.tiles_n = (g.N + C::BN - 1) / C::BN;
  const dim3 grid(unsigned(g.tiles_m * g.tiles_n), unsigned(splits));
  if (mode == GEMM_ACCUM)
    hipLaunchKernelGGL((gemm_bf16_kernel<C, A_KC, B_KC, GEMM_ACCUM>), grid, dim3(NTHREADS), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<C, A_KC, B_KC, GEMM_STORE>), grid, dim3(NTHREADS), 0, s, g);
  return hipGetLastError();
}

using Small = Cfg<128, 128, 32>;
using Mid = Cfg<256, 128, 32, 2>;   // two workgroups per CU
using Large = Cfg<256, 256, 64>;    // pipelined, one workgroup per CU

template <class C>
hipError_t launch_cfg(bool a_kc, bool b_kc, int mode, const GemmArgs& g, int splits,
                      hipStream_t s) {
  if (a_kc && b_kc) return launch<C, true, true>(mode, g, splits, s);
  if (a_kc) return launch<C, true, false>(mode, g, splits, s);
  if (b_kc) return launch<C, false, true>(mode, g, splits, s);
  return launch<C, false, false>(mode, g, splits, s);
}

hipError_t launch_large(bool a_kc, bool b_kc, int mode, const GemmArgs& g, int splits,
                        hipStream_t s) {
  if (a_kc && b_kc) return launch_pipe<Large, true, true>(mode, g, splits, s);
  if (a_kc) return launch_pipe<Large, true, false>(mode, g, splits, s);
  if (b_kc) return launch_pipe<Large, false, true>(mode, g, splits, s);
  return launch_pipe<Large, false, false>(mode, g, splits, s);
}

}  // namespace

hipError_t gemm_bf16(bool a_kcontig, bool b_kcontig, int mode, const GemmArgs& g, int splits,
                     hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  // Tile choice from measurements on MI355X: the pipelined 256 x 256 tile
  // whenever it gives at least two workgroups per CU (MN-contiguous operands
  // read through the LDS transpose); otherwise, with a transposed operand,
  // the 256 x 128 tile at two workgroups per CU, which overlaps one
  // workgroup's staging and barrier with the other's MFMAs; small problems
  // the 128 x 128 tile.
  const int64_t large_tiles = int64_t((g.M + 255) / 256) * ((g.N + 255) / 256) * splits;
  const int64_t mid_tiles = int64_t((g.M + 255) / 256) * ((g.N + 127) / 128) * splits;
  if (large_tiles >= 512) return launch_large(a_kcontig, b_kcontig, mode, g, splits, s);
  if (!(a_kcontig && b_kcontig) && mid_tiles >= 512)
    return launch_cfg<Mid>(a_kcontig, b_kcontig, mode, g, splits, s);
  return launch_cfg<Small>(a_kcontig, b_kcontig, mode, g, splits, s);
}

hipError_t gemm_bf16_logits(const GemmArgs& g0, hipStream_t s) {
  if (g0.M == 0 || g0.N == 0) return hipSuccess;
  GemmArgs g = g0;
  g.vec_c = 0;
  g.tiles_m = (g.M + Large::BM - 1) / Large::BM;
  g.tiles_n = (g.N + Large::BN - 1) / Large::BN;
  const dim3 grid(unsigned(g.tiles_m * g.tiles_n), 1u);
  hipLaunchKernelGGL((gemm_bf16_pipe_kernel<Large, true, true, GEMM_LOGITS>), grid,
                     dim3(NTHREADS), 0, s, g);
  return hipGetLastError();
}

}  // namespace grpo

using namespace grpo;

// C ABI: one GEMM of the fused-linear path, exported for tests and callers
// that want the products on their own (see grpo_rows.h).
extern "C" int grpo_gemm_bf16(const void* A, int a_layout, int64_t lda, const void* B,
                              int b_layout, int64_t ldb, float* C, int64_t ldc, int64_t M,
                              int64_t N, int64_t K, int accumulate, void* stream) {
  if (M < 0 || N < 0 || K < 0 || M > (1 << 30) || N > (1 << 30) || K > (1 << 30))
    return GRPO_ERR_SHAPE;
  // the grid (128 x 128 tiles at the smallest, 256 lanes each) must fit one
  // dispatch's 32-bit work-item count
  if (((M + 127) / 128) * ((N + 127) / 128) > groups_per_launch(256)) return GRPO_ERR_SHAPE;
  if (M == 0 || N == 0) return GRPO_OK;
  if (A == nullptr || B == nullptr || C == nullptr) return GRPO_ERR_NULL;
  if ((a_layout != 0 && a_layout != 1) || (b_layout != 0 && b_layout != 1) ||
      (accumulate != 0 && accumulate != 1))
    return GRPO_ERR_PARAM;
  const bool akc = a_layout == 0, bkc = b_layout == 0;
  // contiguous extents and leading dimensions in whole 16-byte chunks
  if (K % 8 != 0 || (!akc && M % 8 != 0) || (!bkc && N % 8 != 0)) return GRPO_ERR_SHAPE;
  if (lda % 8 != 0 || ldb % 8 != 0) return GRPO_ERR_STRIDE;
  if (lda < (akc ? K : M) || ldb < (bkc ? K : N) || ldc < N) return GRPO_ERR_STRIDE;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 4)) return GRPO_ERR_ALIGN;
  GemmArgs g{};
  g.A = static_cast<const uint16_t*>(A);
  g.lda = lda;
  g.B = static_cast<const uint16_t*>(B);
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  g.M = int32_t(M);
  g.N = int32_t(N);
  g.K = int32_t(K);
  g.k_per_split = int32_t(((K + 63) / 64) * 64);
  if (g.k_per_split == 0) g.k_per_split = 64;
  g.split_stride = 0;
  const hipError_t e = gemm_bf16(akc, bkc, accumulate ? GEMM_ACCUM : GEMM_STORE, g, 1,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GRPO_OK : GRPO_ERR_LAUNCH;
}

// C ABI: the fused chunk's logits product with its statistics epilogue,
// exported for tests and timing (see grpo_rows.h).
extern "C" int grpo_gemm_bf16_logits(const void* A, int64_t lda, const void* B, int64_t ldb,
                                     int64_t M, int64_t N, int64_t K, float temperature,
                                     const int64_t* ids, void* z16, int64_t ldz, float* stat,
                                     float* zy, void* stream) {
  if (M < 0 || N < 0 || K < 0 || M > (1 << 30) || N > (1 << 30) || K > (1 << 30))
    return GRPO_ERR_SHAPE;
  if (((M + 255) / 256) * ((N + 255) / 256) > groups_per_launch(256)) return GRPO_ERR_SHAPE;
  if (!(temperature > 0.0f) || !std::isfinite(temperature)) return GRPO_ERR_PARAM;
  if (M == 0 || N == 0) return GRPO_OK;
  if (A == nullptr || B == nullptr || ids == nullptr || z16 == nullptr || stat == nullptr ||
      zy == nullptr)
    return GRPO_ERR_NULL;
  if (K % 8 != 0 || N % 8 != 0 || K == 0) return GRPO_ERR_SHAPE;
  if (lda % 8 != 0 || ldb % 8 != 0 || ldz % 8 != 0 || lda < K || ldb < K || ldz < N)
    return GRPO_ERR_STRIDE;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(z16, 16) || !aligned(stat, 4) ||
      !aligned(zy, 4) || !aligned(ids, 8))
    return GRPO_ERR_ALIGN;
  GemmArgs g{};
  g.A = static_cast<const uint16_t*>(A);
  g.lda = lda;
  g.B = static_cast<const uint16_t*>(B);
  g.ldb = ldb;
  g.ldc = ldz;
  g.M = int32_t(M);
  g.N = int32_t(N);
  g.K = int32_t(K);
  g.k_per_split = int32_t(((K + 63) / 64) * 64);
  g.z16 = static_cast<uint16_t*>(z16);
  g.stat = stat;
  g.stat_ld = M;
  g.ids = ids;
  g.zy = zy;
  g.cscale = kLog2e / temperature;
  return gemm_bf16_logits(g, static_cast<hipStream_t>(stream)) == hipSuccess ? GRPO_OK
                                                                             : GRPO_ERR_LAUNCH;
}
