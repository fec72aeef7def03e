/*
 * grpo_rows.h -- C ABI of the MI355X (gfx950) row-wise GRPO logits library.
 *
 * The library computes, over LM-head logits laid out as N = B*L rows of V
 * vocabulary entries, the per-row work of GRPO fine-tuning: a temperature-
 * scaled log-sum-exp, the log-softmax of the sampled token, the entropy, the
 * per-token GRPO loss (PPO clipped-ratio surrogate plus beta * k3 KL against a
 * reference log-probability), and the backward
 *     dlogits = dlogp * (onehot(y) - softmax(z / T)) / T
 * with an all-zero, write-only path for rows whose dlogp is exactly 0.
 * A chunked fused-linear entry point forms the logits of one batch chunk from
 * hidden states and the LM-head weight, and accumulates the gradients of both
 * during the forward, so the full logits are never held.
 *
 * Sources (web pages, cited by title and section):
 *   [LIGER-BWD] Liger-Kernel PR #1550 analysis, "GRPO loss backward
 *               optimisation": "Code analysis" (the _grpo_loss_bwd_kernel and
 *               _grpo_loss_bwd_kernel_seq hunks) and "Why is this good".
 *   [LIGER-TRL] "Liger GRPO meets TRL" summary, detailed items 3 and 4.
 *   [AXOLOTL]   axolotl PR #3510 analysis, "entropy and selective log-softmax
 *               with Triton kernels", "Code analysis" parts 1 and 2.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Ownership: every array argument is a DEVICE pointer owned by the caller.
 *    The library never allocates, frees or copies device memory; the fused
 *    path uses only the workspace the caller passes, or, in
 *    fused_linear_grpo_chunk_noalloc, a static device array of the library's
 *    own.  Parameter structs are host pointers, read during the call only.
 *  - Layout: logits are row-major [rows, ld] with row r at logits + r*ld
 *    elements and the first V entries of each row used (ld >= V; a slice of a
 *    wider buffer is allowed).  Row r of a GRPO batch is token t of sequence
 *    b with r = b*L + t.  Per-row arrays are dense [B*L]; per-sequence arrays
 *    are dense [B].
 *  - dtype: GRPO_F32 (float) or GRPO_BF16 (bfloat16 bit patterns, uint16).
 *    Arithmetic is fp32 with fp32 accumulation.  dlogits has the logits'
 *    dtype; bf16 results are rounded to nearest even.
 *  - Execution: all work is enqueued asynchronously on `stream` (a
 *    hipStream_t; NULL is the default stream).  No call synchronises.
 *  - Errors: argument errors are detected on the host and returned before
 *    anything is enqueued (no device is touched).  A launch failure returns
 *    GRPO_ERR_LAUNCH.  Data errors are not status codes (that would need a
 *    sync): an id outside [0, V) makes that row's outputs NaN and, where an
 *    err_count pointer is given, adds 1 to it with a device atomic.
 *    NaN/Inf in the logits propagate to the outputs of their row; finite
 *    logits must lie above -1e30 (the normaliser's starting value).
 *  - Alignment: pointers must be aligned to their element size.  Rows whose
 *    byte address is 16-byte aligned take 128-bit loads and stores; other
 *    layouts take an element-wise path with the same results.
 *  - Aliasing: dlogits may alias logits only with the same dtype and
 *    ld_out == ld (in place).  No other output may alias an input.
 *  - Limits: up to 2^31 - 1 rows and 2^26 columns per call.  A dispatch
 *    covers at most 2^32 - 1 work-items, so the row kernels (and the fused
 *    chunk's row gather and split-K reduction) run as several launches where
 *    a call needs more; the matrix products, whose tiles cannot be split
 *    that way, return GRPO_ERR_SHAPE past 2^32 - 1 work-items (16777215
 *    tiles of 256 lanes).
 *  - Thread safety: reentrant; every call may run from any host thread.
 *    The row kernels keep no state.  The exception is fused_linear_grpo_chunk,
 *    which keeps one side stream per device for the process (default
 *    priority, made on its first call there, guarded by a mutex) and creates
 *    and destroys a pair of events per call to fork to and join from it.
 *    rows == 0 is a no-op.
 */
#ifndef GRPO_ROWS_H
#define GRPO_ROWS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum grpo_status {
  GRPO_OK = 0,
  GRPO_ERR_NULL = 1,      /* a required pointer is NULL                      */
  GRPO_ERR_SHAPE = 2,     /* B, L, V, rows, H out of range                   */
  GRPO_ERR_STRIDE = 3,    /* ld < V or ld_out < V                            */
  GRPO_ERR_DTYPE = 4,     /* dtype not GRPO_F32 / GRPO_BF16                  */
  GRPO_ERR_ALIGN = 5,     /* pointer not aligned to its element size         */
  GRPO_ERR_WORKSPACE = 6, /* fused-linear workspace NULL or too small        */
  GRPO_ERR_LAUNCH = 7,    /* the HIP runtime refused a launch                */
  GRPO_ERR_PARAM = 8,     /* temperature <= 0, eps out of range, bad level   */
  GRPO_ERR_SCRATCH = 9    /* chunk needs more than the no-alloc scratch      */
};

enum grpo_dtype { GRPO_F32 = 0, GRPO_BF16 = 1 };
enum grpo_level { GRPO_TOKEN = 0, GRPO_SEQUENCE = 1 };

/* flags: GRPO_FLAG_FORCE_DENSE makes the backward take the dense path on every
 * row (the all-zero path is skipped even when dlogp == 0); results are equal
 * to the default up to the sign of zero.  Used to check the early path. */
enum grpo_flags { GRPO_FLAG_FORCE_DENSE = 1u };

/* Loss settings.  temperature T > 0 divides the logits before the softmax
 * [LIGER-BWD, "Code analysis": division by TEMPERATURE].  beta >= 0 weighs the
 * k3 KL term (beta = 0 drops it) [same passage: BETA].  The ratio is clipped
 * to [1 - eps_low, 1 + eps_high] (0 <= eps_low < 1, eps_high >= 0).  level is
 * GRPO_TOKEN (one ratio per token) or GRPO_SEQUENCE (one ratio per sequence,
 * from the mask-weighted mean log-ratio) [LIGER-BWD: _grpo_loss_bwd_kernel
 * and _grpo_loss_bwd_kernel_seq]. */
typedef struct grpo_params {
  float temperature;
  float beta;
  float eps_low;
  float eps_high;
  int32_t level;
  uint32_t flags;
} grpo_params;

/* ------------------------------------------------------------------------
 * grpo_logits_fwd -- forward row pass of the GRPO loss.
 * Defines: per row r, u = z_r / T, lse = log sum_j e^{u_j},
 *   logp = u_y - lse, entropy = -sum_j p_j log p_j, x = logp - old_logp,
 *   ratio = e^x, pg = -min(ratio*A, clip(ratio, 1-eps_low, 1+eps_high)*A),
 *   kl = e^d - d - 1 with d = ref_logp - logp, loss = pg + beta*kl.
 * [LIGER-BWD "Code analysis": the backward consumes logp, ref_logp, BETA and
 *  the PPO-clipped flag; AXOLOTL part 1 (entropy), part 2 (selective
 *  log-softmax)].  At GRPO_SEQUENCE, x is averaged over the valid tokens of
 *  each sequence (mask-weighted, divided by max(count, 1)), ratio = e^{mean}
 *  is written to seq_ratio[b] and pg is that sequence's, broadcast to all of
 *  its tokens; the KL term stays per token.
 *
 * logits     [B*L, ld] of `dtype`            (in)
 * ids        int64 [B*L] sampled token ids   (in)
 * old_logp   fp32 [B*L]                      (in)
 * ref_logp   fp32 [B*L] or NULL: NULL means no reference model (ref equals
 *            the policy, kl = 0)             (in)
 * adv        fp32 [B] advantage per sequence (in)
 * mask       uint8 [B*L] completion mask or NULL (all ones; a nonzero entry
 *            counts as 1); used only at
 *            GRPO_SEQUENCE (per-token losses are reported for every token;
 *            the caller's reduction applies the mask)  (in)
 * loss, logp, lse  fp32 [B*L]                (out, required)
 * entropy, kl      fp32 [B*L] or NULL        (out, optional)
 * is_clipped uint8 [B*L] or NULL: 1 where the clipped branch is strictly the
 *            smaller one (per sequence at GRPO_SEQUENCE)  (out, optional)
 * gathered   fp32 [B*L] or NULL: z[r, ids[r]] upcast exactly  (out, optional)
 * seq_ratio  fp32 [B]: required iff level == GRPO_SEQUENCE, else ignored (out)
 * err_count  int32 [1] or NULL: += number of rows with an id outside [0, V)
 * ------------------------------------------------------------------------ */
int grpo_logits_fwd(const void* logits, int dtype, int64_t B, int64_t L, int64_t V,
                    int64_t ld, const int64_t* ids, const float* old_logp,
                    const float* ref_logp, const float* adv, const uint8_t* mask,
                    const grpo_params* p, float* loss, float* logp, float* lse,
                    float* entropy, float* kl, uint8_t* is_clipped, float* gathered,
                    float* seq_ratio, int32_t* err_count, void* stream);

/* ------------------------------------------------------------------------
 * grpo_logits_bwd -- backward of sum_r dloss[r] * loss[r] w.r.t. the logits.
 * Defines [LIGER-BWD "Code analysis", both kernels; "Why is this good"]:
 *   token:    g = (-ratio*A*[not clipped] + beta*(1 - e^{ref - logp})) * dloss
 *   sequence: g = -ratio_b*A_b*[not clipped_b] * (sum_t' dloss_bt') * m_bt/n_b
 *                 + beta*(1 - e^{ref - logp}) * dloss_bt,  n_b = max(sum_t m, 1)
 *   dlogits_j = g/T * (1[j == y] - e^{u_j - lse}).
 * A row with g == 0 (zero advantage with no KL gradient, PPO-clipped token
 * with beta == 0, or dloss == 0) is written as +0.0 without reading its
 * logits.  ratio and the clipped flag are recomputed from logp and old_logp
 * (token) or taken from seq_ratio (sequence) exactly as the forward did.
 *
 * logits, ids, old_logp, ref_logp, adv, mask, p: as for grpo_logits_fwd (in)
 * logp, lse  fp32 [B*L] from grpo_logits_fwd (in, required)
 * seq_ratio  fp32 [B] from grpo_logits_fwd; required iff GRPO_SEQUENCE (in)
 * dloss      fp32 [B*L] upstream gradient of each token's loss (in)
 * dlogits    [B*L, ld_out] of `dtype` (out); may alias logits if ld_out == ld
 * zero_row   uint8 [B*L] or NULL: 1 where the row took the all-zero path
 *            (that is, g == 0), even under GRPO_FLAG_FORCE_DENSE  (out)
 * Rows with an id outside [0, V) are written as NaN.
 * ------------------------------------------------------------------------ */
int grpo_logits_bwd(const void* logits, int dtype, int64_t B, int64_t L, int64_t V,
                    int64_t ld, const int64_t* ids, const float* old_logp,
                    const float* ref_logp, const float* adv, const uint8_t* mask,
                    const grpo_params* p, const float* logp, const float* lse,
                    const float* seq_ratio, const float* dloss, void* dlogits,
                    int64_t ld_out, uint8_t* zero_row, void* stream);

/* ------------------------------------------------------------------------
 * grpo_logits_fwd_bwd -- forward and backward of the token-level loss in a
 * single pass, for callers that know the per-token upstream weight dloss
 * before the forward (a token-mean or sum reduction of the per-token loss;
 * the chunked loss of [LIGER-TRL] items 3-4 computes gradients during the
 * forward in the same way).  Computes exactly what grpo_logits_fwd followed
 * by grpo_logits_bwd compute (same definitions, same early all-zero rows),
 * but each row is read once into registers and dlogits written from them.
 * Rows longer than 128 KB, or not 16-byte aligned, take the two-pass path
 * internally (then dlogits may not alias logits).  level must be
 * GRPO_TOKEN (GRPO_ERR_PARAM otherwise).
 *
 * Arguments as grpo_logits_fwd / grpo_logits_bwd: logits, ids, old_logp,
 * ref_logp (nullable), adv, mask (unused at token level), p, dloss (in);
 * loss, logp, lse (out, required); entropy, kl, is_clipped (out, nullable);
 * dlogits [B*L, ld_out] of `dtype` (out; may alias logits if ld_out == ld
 * and the row fits in registers); zero_row (out, nullable); err_count
 * (nullable).
 * ------------------------------------------------------------------------ */
int grpo_logits_fwd_bwd(const void* logits, int dtype, int64_t B, int64_t L, int64_t V,
                        int64_t ld, const int64_t* ids, const float* old_logp,
                        const float* ref_logp, const float* adv, const uint8_t* mask,
                        const grpo_params* p, const float* dloss, float* loss, float* logp,
                        float* lse, float* entropy, float* kl, uint8_t* is_clipped,
                        void* dlogits, int64_t ld_out, uint8_t* zero_row, int32_t* err_count,
                        void* stream);

/* ------------------------------------------------------------------------
 * entropy_from_logits -- per-row entropy of softmax(z / temperature).
 * Defines [AXOLOTL part 1: minus the row sum of exp(logp) * logp of the row
 * log-softmax; strided rows read in place].  temperature 1 is the plain op.
 * logits [rows, ld] (in); entropy fp32 [rows] (out).  A row containing -inf
 * has entropy NaN, as the definition's 0 * (-inf) gives.
 * ------------------------------------------------------------------------ */
int entropy_from_logits(const void* logits, int dtype, int64_t rows, int64_t V, int64_t ld,
                        float temperature, float* entropy, void* stream);

/* ------------------------------------------------------------------------
 * selective_log_softmax -- logp[r] = log_softmax(z_r / T)[ids[r]].
 * Defines [AXOLOTL part 2].  logits [rows, ld], ids int64 [rows] (in);
 * logp fp32 [rows] (out); lse fp32 [rows] or NULL (out; needed by the
 * backward).  An id outside [0, V) gives NaN.
 * ------------------------------------------------------------------------ */
int selective_log_softmax(const void* logits, int dtype, int64_t rows, int64_t V, int64_t ld,
                          const int64_t* ids, float temperature, float* logp, float* lse,
                          void* stream);

/* ------------------------------------------------------------------------
 * selective_log_softmax_bwd -- custom backward of selective_log_softmax:
 *   dlogits_j = grad_logp[r] / T * (1[j == ids[r]] - e^{z_j/T - lse[r]}).
 * Defines [AXOLOTL part 2: the custom autograd backward].  Rows with
 * grad_logp == 0 take the all-zero, write-only path.
 * logits [rows, ld], ids, lse (from the forward), grad_logp fp32 [rows] (in);
 * dlogits [rows, ld_out] of `dtype` (out; may alias logits if ld_out == ld).
 * ------------------------------------------------------------------------ */
int selective_log_softmax_bwd(const void* logits, int dtype, int64_t rows, int64_t V,
                              int64_t ld, const int64_t* ids, float temperature,
                              const float* lse, const float* grad_logp, void* dlogits,
                              int64_t ld_out, void* stream);

/* ------------------------------------------------------------------------
 * fused_linear_grpo_chunk -- one batch chunk of the chunked fused-linear
 * GRPO loss, gradients taken during the forward [LIGER-TRL items 3-4].
 * For the chunk's R = nseq*L rows:
 *   z = hidden * weight^T (fp32 accumulation; never the whole batch),
 *   token-level GRPO forward + backward of sum dloss*loss on z,
 *   *loss_accum += sum_r dloss[r] * loss[r],
 *   grad_hidden = dz * weight            (overwritten, fp32 [R, H]),
 *   grad_weight += dz^T * hidden         (accumulated, fp32 [V, H]).
 * The forward (softmax statistics, logp, loss) works from the fp32 values
 * of z; the backward's softmax reads z rounded to bf16 (kept in the
 * workspace), and dz is bf16 for the two products.  The caller loops over
 * chunks; level must be GRPO_TOKEN.  Rows whose dloss is exactly 0 (padding,
 * masked tokens) add nothing to any output and are not computed: they are
 * compacted away on the device before the first product (the zero-gradient
 * skip of [LIGER-BWD "Why is this good"] applied to the chunk), their
 * grad_hidden rows are written as 0, and non-finite inputs on them do not
 * propagate.  mask is not read (dloss carries it at token level).
 *
 * hidden bf16 [R, H] row-major; weight bf16 [V, H] row-major (in)
 * ids, old_logp, ref_logp (nullable), mask (nullable), dloss: [R] (in)
 * adv fp32 [nseq] (in)
 * loss_accum fp32 [1] (in/out, device); grad_hidden fp32 [R, H] (out);
 * grad_weight fp32 [V, H] (in/out)
 * workspace: device buffer of at least
 *   fused_linear_grpo_workspace_bytes(R, V, H) bytes, 256-byte aligned; it
 *   holds the chunk's bf16 logits, overwritten by its bf16 dlogits (2 R V
 *   bytes), the per-row softmax statistics (8 R bytes per 128 columns of
 *   V, later reused for grad_hidden's split-K partial sums) and the
 *   compacted rows' hidden states and inputs (about 2 R H + 36 R).
 * H must be a multiple of 64 and at most 65536; V a multiple of 8 and at
 * most 2^30; R = nseq * L at most 2^30 (GRPO_ERR_SHAPE otherwise).  hidden,
 * weight and grad_hidden 16-byte aligned.  The result is deterministic.
 * grad_weight's product runs on a stream the library keeps per device
 * (default priority, made on the first call), forked from and joined back
 * into `stream` within the call, so work enqueued on `stream` afterwards
 * sees every output complete.
 * ------------------------------------------------------------------------ */
int fused_linear_grpo_chunk(const void* hidden, int64_t nseq, int64_t L, int64_t H,
                            const void* weight, int64_t V, const int64_t* ids,
                            const float* old_logp, const float* ref_logp, const float* adv,
                            const uint8_t* mask, const float* dloss, const grpo_params* p,
                            float* loss_accum, float* grad_hidden, float* grad_weight,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fused_linear_grpo_chunk needs for R rows (0 on bad sizes). */
size_t fused_linear_grpo_workspace_bytes(int64_t rows, int64_t V, int64_t H);

/* ------------------------------------------------------------------------
 * fused_linear_grpo_chunk_noalloc -- fused_linear_grpo_chunk for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, results
 * and determinism as fused_linear_grpo_chunk (bit-identical outputs), minus
 * the workspace: the chunk's workspace is a static device array of the
 * library's own, 384 MiB (402653184 bytes), of which each device that calls
 * this entry point holds one copy until the process ends.  Every step runs
 * on `stream` (no side stream, no events): the call creates and allocates
 * nothing.
 * Limit: fused_linear_grpo_workspace_bytes(nseq*L, V, H) <= 402653184 (one
 * 1024-token sequence at V = 151936, H = 1024 needs about 363 MiB); a larger
 * chunk returns GRPO_ERR_SCRATCH before anything is enqueued.
 * Concurrency: all calls on one device share its array, and nothing of it
 * needs to start zeroed (every step writes what a later one reads), so calls
 * ordered on one stream are safe; calls that overlap on one device (other
 * streams, other host threads) race on the array and give wrong results.
 * Other errors as for fused_linear_grpo_chunk; GRPO_ERR_LAUNCH also when the
 * runtime cannot give the array's device address.
 * ------------------------------------------------------------------------ */
int fused_linear_grpo_chunk_noalloc(const void* hidden, int64_t nseq, int64_t L, int64_t H,
                                    const void* weight, int64_t V, const int64_t* ids,
                                    const float* old_logp, const float* ref_logp,
                                    const float* adv, const uint8_t* mask, const float* dloss,
                                    const grpo_params* p, float* loss_accum, float* grad_hidden,
                                    float* grad_weight, void* stream);

/* ------------------------------------------------------------------------
 * grpo_gemm_bf16 -- the bf16 matrix-core product the fused-linear path is
 * built from, exported on its own:  C[M, N] (=, or += with accumulate = 1)
 *   sum_k A[m, k] B[k, n],  fp32 accumulation and output.
 * a_layout 0: A[m, k] at A + m*lda + k (K-contiguous); 1: at A + k*lda + m.
 * b_layout 0: B[k, n] at B + n*ldb + k (K-contiguous); 1: at B + k*ldb + n.
 * A, B bf16, 16-byte aligned, lda and ldb multiples of 8; K, and M (N) when A
 * (B) is not K-contiguous, multiples of 8.  C fp32 row-major with ldc >= N.
 * [LIGER-TRL items 3-4: the chunk's logits h W^T and the gradients dz W and
 *  dz^T h are these three products.]
 * ------------------------------------------------------------------------ */
int grpo_gemm_bf16(const void* A, int a_layout, int64_t lda, const void* B, int b_layout,
                   int64_t ldb, float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                   int accumulate, void* stream);

/* ------------------------------------------------------------------------
 * grpo_gemm_bf16_logits -- the fused-linear chunk's logits product in the
 * form the chunk runs it, exported so it can be tested and timed alone
 * [LIGER-TRL items 3-4: the chunk's logits h W^T; the forward's row
 * statistics taken from them]:  z = A B^T with K-contiguous A [M, K] (lda)
 * and B [N, K] (ldb), fp32 accumulation, then from the fp32 values
 *   z16[r, n]   = bf16(z[r, n])  (round to nearest even; leading dim ldz),
 *   for each row r and 128-column half p = 0 .. P-1, P = 2 ceil(N / 256):
 *     stat[p*M + r]       = m = max of z[r, n] over n in [128p, 128p+128) and < N,
 *     stat[(P + p)*M + r] = sum of exp((z[r, n] - m) / T) over those n
 *     (m = -1e30 and the sum 0 when the half holds no column),
 *   zy[r] = z[r, ids[r]] when 0 <= ids[r] < N (else zy[r] is not written).
 * Merging a row's P partials gives its log-sum-exp of z / T.
 * A, B, z16 bf16 and 16-byte aligned; lda, ldb, ldz multiples of 8 with
 * lda, ldb >= K and ldz >= N; K and N multiples of 8; ids int64 [M]; stat
 * fp32 [2 P M]; zy fp32 [M]; temperature > 0 and finite.
 * ------------------------------------------------------------------------ */
int grpo_gemm_bf16_logits(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M,
                          int64_t N, int64_t K, float temperature, const int64_t* ids,
                          void* z16, int64_t ldz, float* stat, float* zy, void* stream);

/* ------------------------------------------------------------------------
 * entropy_from_logits_bwd -- backward of the per-row entropy
 * H = -sum_j p_j log p_j, p = softmax(z / T) [AXOLOTL part 1 defines H; the
 * pages give it no backward, so this is its derivative]:
 *   dlogits_j = -grad_entropy[r] / T * p_j * (log p_j + H[r]),
 *   log p_j = z_j / T - lse[r],
 * for entropy-regularised losses.  Rows with grad_entropy == 0 take the
 * all-zero, write-only path (no logits read).
 * logits [rows, ld] (in); lse, entropy fp32 [rows] (in: the forward's, at the
 * same T -- grpo_logits_fwd writes both); grad_entropy fp32 [rows] (in);
 * dlogits [rows, ld_out] of `dtype` (out; may alias logits if ld_out == ld).
 * Errors as for selective_log_softmax_bwd.
 * ------------------------------------------------------------------------ */
int entropy_from_logits_bwd(const void* logits, int dtype, int64_t rows, int64_t V, int64_t ld,
                            float temperature, const float* lse, const float* entropy,
                            const float* grad_entropy, void* dlogits, int64_t ld_out,
                            void* stream);

/* ------------------------------------------------------------------------
 * grpo_group_advantages -- group-relative advantages of n rewards in
 * consecutive groups of group_size (the completions of one prompt):
 *   A = (r - mean_group) / (sample_std_group + eps)   (scale = 1),
 *   A =  r - mean_group                                (scale = 0).
 * The pages name zero-advantage sequences [LIGER-BWD summary] but give no
 * formula; this is the plain reading of "group-relative", with the sample
 * (n - 1) standard deviation.  A group whose rewards are all equal (or a
 * group of one) gets exactly 0 -- the rows the zero-gradient path skips.
 * Sums are taken in fp64; a NaN reward makes its group NaN.
 * rewards, adv fp32 [n] (in, out).  n % group_size == 0 (else
 * GRPO_ERR_SHAPE); eps >= 0 and scale in {0, 1} (else GRPO_ERR_PARAM).
 * ------------------------------------------------------------------------ */
int grpo_group_advantages(const float* rewards, int64_t n, int64_t group_size, float eps,
                          int scale, float* adv, void* stream);

/* Reductions of the per-token losses for grpo_loss_weights. */
enum { GRPO_REDUCE_TOKEN = 0, GRPO_REDUCE_SEQUENCE = 1, GRPO_REDUCE_CONSTANT = 2 };

/* ------------------------------------------------------------------------
 * grpo_loss_weights -- the per-token weights dloss = dLoss/dloss_bt that the
 * backward entry points take [LIGER-BWD "Code analysis": the backward scales
 * by dloss], for three reductions of the per-token losses l (m = mask, all
 * ones when mask is NULL; the pages do not fix the reduction):
 *   GRPO_REDUCE_TOKEN     Loss = sum m l / max(sum m, 1)
 *   GRPO_REDUCE_SEQUENCE  Loss = (1/B) sum_b sum_t m l / max(n_b, 1)
 *   GRPO_REDUCE_CONSTANT  Loss = sum m l / (B L)
 * Counts are exact integers; each weight is the correctly rounded fp32 of
 * its reciprocal.  mask uint8 [B*L] or NULL (in); dloss fp32 [B*L] (out).
 * ------------------------------------------------------------------------ */
int grpo_loss_weights(const uint8_t* mask, int64_t B, int64_t L, int reduction, float* dloss,
                      void* stream);

/* Static, NUL-terminated description of a status code. */
const char* grpo_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GRPO_ROWS_H */
