// gemm_mfma.hip -- bf16 MFMA GEMM for the chunked fused-linear loss (see
// gemm_mfma.hpp for the layouts, tiling and fragment layout).
#include <hip/hip_runtime.h>

#include "gemm_mfma.hpp"
#include "grpo_rows.h"
#include "host_common.hpp"

namespace grpo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LROW = BK + 8;  // LDS row pitch in bf16 (80 bytes: 16-byte pad)
constexpr int NTHREADS = 256;

// Stage one operand tile (ROWS x BK, rows = M or N index) into registers.
// K-contiguous: lane t loads chunks t and t + 256 (row = c / 4, 8 k each).
// MN-contiguous: lane t loads K-rows 2q, 2q+1 (q = t % 4) of the 8 x 8 block
// t / 4 (4 K-blocks x 16 row-blocks).
template <bool KC>
__device__ __forceinline__ void stage_load(const uint16_t* __restrict__ P, int64_t ld, int extent,
                                           int r0, int k0, int kend, v4u (&v)[2]) {
  const int t = threadIdx.x;
  if constexpr (KC) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = t + NTHREADS * i;
      const int row = c >> 2, kc = (c & 3) * 8;
      const bool ok = (r0 + row < extent) && (k0 + kc < kend);
      v[i] = ok ? *reinterpret_cast<const v4u*>(P + int64_t(r0 + row) * ld + k0 + kc)
                : v4u{0u, 0u, 0u, 0u};
    }
  } else {
    const int b = t >> 2, q = t & 3;
    const int kb = b >> 4, rb = b & 15;
    const bool col_ok = r0 + rb * 8 < extent;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = k0 + kb * 8 + 2 * q + i;
      const bool ok = col_ok && (k < kend);
      v[i] = ok ? *reinterpret_cast<const v4u*>(P + int64_t(k) * ld + r0 + rb * 8)
                : v4u{0u, 0u, 0u, 0u};
    }
  }
}

// Write staged registers to an LDS tile laid out [row][k] with pitch LROW.
template <bool KC>
__device__ __forceinline__ void stage_store(uint16_t* __restrict__ lds, const v4u (&v)[2]) {
  const int t = threadIdx.x;
  if constexpr (KC) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = t + NTHREADS * i;
      const int row = c >> 2, kc = (c & 3) * 8;
      *reinterpret_cast<v4u*>(lds + row * LROW + kc) = v[i];
    }
  } else {
    const int b = t >> 2, q = t & 3;
    const int kb = b >> 4, rb = b & 15;
    uint32_t* base = reinterpret_cast<uint32_t*>(lds + (rb * 8) * LROW + kb * 8 + 2 * q);
    const uint32_t x[4] = {v[0].x, v[0].y, v[0].z, v[0].w};  // K-row 2q, 8 rows' values
    const uint32_t y[4] = {v[1].x, v[1].y, v[1].z, v[1].w};  // K-row 2q + 1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // element 2j (low halves) and 2j + 1 (high halves) of both K-rows
      base[(2 * j) * (LROW / 2)] = __builtin_amdgcn_perm(y[j], x[j], 0x05040100u);
      base[(2 * j + 1) * (LROW / 2)] = __builtin_amdgcn_perm(y[j], x[j], 0x07060302u);
    }
  }
}

template <bool A_KC, bool B_KC, int MODE>
__global__ __launch_bounds__(NTHREADS) void gemm_bf16_kernel(GemmArgs g) {
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

  const int z = blockIdx.y;
  const int kbeg = z * g.k_per_split;
  const int kend = min(g.K, kbeg + g.k_per_split);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;

  v4u ra[2], rb[2];
  stage_load<A_KC>(g.A, g.lda, g.M, m0, kbeg, kend, ra);
  stage_load<B_KC>(g.B, g.ldb, g.N, n0, kbeg, kend, rb);
  stage_store<A_KC>(As[0], ra);
  stage_store<B_KC>(Bs[0], rb);
  __syncthreads();

  int buf = 0;
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) {
      stage_load<A_KC>(g.A, g.lda, g.M, m0, k0 + BK, kend, ra);
      stage_load<B_KC>(g.B, g.ldb, g.N, n0, k0 + BK, kend, rb);
    }
    const uint16_t* a_l = As[buf] + (wm * 64 + (lane & 31)) * LROW + 8 * (lane >> 5);
    const uint16_t* b_l = Bs[buf] + (wn * 64 + (lane & 31)) * LROW + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = *reinterpret_cast<const bf16x8*>(a_l + i * 32 * LROW + s * 16);
        fb[i] = *reinterpret_cast<const bf16x8*>(b_l + i * 32 * LROW + s * 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[jj], acc[i][jj], 0, 0, 0);
    }
    if (more) {
      stage_store<A_KC>(As[buf ^ 1], ra);
      stage_store<B_KC>(Bs[buf ^ 1], rb);
    }
    __syncthreads();
    buf ^= 1;
  }

  float* C = g.C + int64_t(z) * g.split_stride;
  const int nl = lane & 31, mg = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int n = n0 + wn * 64 + jj * 32 + nl;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + mg + (r & 3);
        if (m < g.M) {
          float* p = C + int64_t(m) * g.ldc + n;
          if constexpr (MODE == GEMM_ACCUM) *p += acc[i][jj][r];
          else *p = acc[i][jj][r];
        }
      }
    }
  }
}

template <bool A_KC, bool B_KC>
hipError_t launch(int mode, const GemmArgs& g, int splits, hipStream_t s) {
  const dim3 grid(unsigned(g.tiles_m * g.tiles_n), unsigned(splits));
  if (mode == GEMM_ACCUM)
    hipLaunchKernelGGL((gemm_bf16_kernel<A_KC, B_KC, GEMM_ACCUM>), grid, dim3(NTHREADS), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<A_KC, B_KC, GEMM_STORE>), grid, dim3(NTHREADS), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16(bool a_kcontig, bool b_kcontig, int mode, const GemmArgs& g_in, int splits,
                     hipStream_t s) {
  GemmArgs g = g_in;
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + BN - 1) / BN;
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (a_kcontig && b_kcontig) return launch<true, true>(mode, g, splits, s);
  if (a_kcontig) return launch<true, false>(mode, g, splits, s);
  if (b_kcontig) return launch<false, true>(mode, g, splits, s);
  return launch<false, false>(mode, g, splits, s);
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
  g.k_per_split = int32_t(((K + 31) / 32) * 32);
  if (g.k_per_split == 0) g.k_per_split = 32;
  g.split_stride = 0;
  const hipError_t e = gemm_bf16(akc, bkc, accumulate ? GEMM_ACCUM : GEMM_STORE, g, 1,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GRPO_OK : GRPO_ERR_LAUNCH;
}
