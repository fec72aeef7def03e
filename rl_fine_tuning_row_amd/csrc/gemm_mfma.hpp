// gemm_mfma.hpp -- bf16 x bf16 -> fp32 GEMM on gfx950 matrix cores.
//
// C[M, N] (=, += or split-K partial) = sum_k A[m, k] B[k, n].
// A is either K-contiguous (A[m, k] at A + m*lda + k) or M-contiguous
// (A + k*lda + m); B is either K-contiguous (B + n*ldb + k) or N-contiguous
// (B + k*ldb + n).  The three products of the chunked fused-linear loss use
// three of these layouts:
//   logits       = h  W^T : A = h  [R, H]  K-contig, B = W [V, H] K-contig
//   grad_hidden  = dz W   : A = dz [R, V]  K-contig, B = W [V, H] N-contig
//   grad_weight += dz^T h : A = dz [R, V]  M-contig, B = h [R, H] N-contig
// (the logits product runs in GEMM_LOGITS mode: no fp32 C; the epilogue
// turns the fp32 accumulators into per-row softmax partials, the target
// logit and a bf16 copy of the logits).
//
// Three block tiles, all 256 lanes = 4 waves in a 2 x 2 grid:
//  * 256 x 256 x 64, software-pipelined (each wave 128 x 128 = 4 x 4
//    v_mfma_f32_32x32x16_bf16, 256 accumulators per lane in AGPRs, one wave
//    per SIMD, 144 KB of LDS), used in every layout once a problem has at
//    least 512 such tiles (all three products of the fused path);
//  * 256 x 128 x 32 at two workgroups per CU for mid-size products with a
//    transposed operand;
//  * 128 x 128 x 32 for small problems.
// Tiles are staged global -> registers -> LDS, double buffered: the next
// K step's global loads are in flight while the current one feeds the
// MFMAs (in the pipelined tile the loads run two steps ahead, spread chunk
// by chunk over the step).  In the pipelined tile a K-contiguous operand
// sits in LDS as [row][k] (16-byte pad; a fragment is one 128-bit read) and
// an MN-contiguous one as [k][row], copied as is and read back transposed
// by ds_read_b64_tr_b16 (two per fragment).  The two smaller tiles keep every
// operand K-contiguous in LDS and transpose an MN-contiguous one while
// staging it: each lane loads two K-rows of an 8 x 8 block and writes 8
// (k, k+1) pairs (one v_perm_b32 each).
//
// Operand fragment layout of v_mfma_f32_32x32x16_bf16 (checked on MI355X):
// lane l holds A[l % 32][8 (l / 32) + j] and B[8 (l / 32) + j][l % 32],
// j = 0..7; accumulator i of lane l is D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grpo {

// GEMM_LOGITS (the chunked loss's logits, both operands K-contiguous):
// C itself is not written; the epilogue keeps the fp32 accumulators for
// per-row softmax statistics and the target logit, and writes C as bf16.
enum GemmMode : int32_t { GEMM_STORE = 0, GEMM_ACCUM = 1, GEMM_LOGITS = 2 };

struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
  int32_t M, N, K;
  int32_t k_per_split;     // multiple of 64; split z covers [z*kps, min(K, (z+1)*kps))
  int64_t split_stride;    // elements between the split-K partial slabs of C
  int32_t tiles_m, tiles_n;
  int32_t vec_c;           // C rows can take 16-byte accesses (set at launch)
  const int32_t* dev_m;    // nullable: M is min(M, *dev_m), read on the device
  const int32_t* dev_k;    // nullable: K is min(K, *dev_k), read on the device
  // GEMM_LOGITS only.  Row r's softmax statistics over the 128-column half
  // p of block column tn (p = 2 tn + h, P = 2 tiles_n halves) are written as
  // m = stat[p*stat_ld + r] and s = stat[(P + p)*stat_ld + r] (the Stat
  // fields of the row kernels with cscale = log2(e)/T; no entropy sum);
  // zy[r] = C[r][ids[r]] in fp32 when ids[r] is a column of C; z16 = C as
  // bf16 with leading dimension ldc.
  uint16_t* z16;
  float* stat;
  int64_t stat_ld;
  const int64_t* ids;
  float* zy;
  float cscale;
};

// Enqueue one GEMM; requires K, and the contiguous extent of every operand,
// to be multiples of 8 (16-byte chunks), lda/ldb multiples of 8, 16-byte
// aligned A and B.  splits > 1 writes partial sums to C + z * split_stride.
// With dev_m / dev_k the host's M / K are upper bounds (the grid is sized
// for them) and the device reads the actual extent: rows of C past it are
// not written, K past it is not summed.  A device K must keep the
// K-contiguous operands' K a multiple of 8 (an MN-contiguous operand takes
// any K).
hipError_t gemm_bf16(bool a_kcontig, bool b_kcontig, int mode, const GemmArgs& g, int splits,
                     hipStream_t s);

// The logits product of the chunked loss (GEMM_LOGITS, K-contiguous A and B,
// no split): always the pipelined 256 x 256 tile; N % 8 == 0, ldc % 8 == 0
// and z16 16-byte aligned.  It writes logits_halves(N) partial statistics
// (two floats each) per row.
hipError_t gemm_bf16_logits(const GemmArgs& g, hipStream_t s);
inline int logits_halves(int64_t N) { return 2 * int((N + 255) / 256); }

}  // namespace grpo
