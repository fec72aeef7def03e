"""Plain float64 definitions of the row-wise GRPO logits pass (NumPy).

TEST INFRASTRUCTURE ONLY: used by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark; never by the HIP library.

Every function is the textbook definition written out, in float64, on the
exact (upcast) input values: two-pass softmax per row, no blocking, no fusion.
Sources (web pages, cited by title and section):

* [LIGER-BWD]  Liger-Kernel PR #1550 analysis, "GRPO loss backward
  optimisation": section "Code analysis" (the ``_grpo_loss_bwd_kernel`` and
  ``_grpo_loss_bwd_kernel_seq`` hunks) and section "Why is this good".
* [LIGER-TRL]  "Liger GRPO meets TRL" summary: detailed summary items 3 and 4
  (chunked LM-head input, gradients of the input chunk and of the LM-head
  weight computed during the forward and accumulated).
* [AXOLOTL]    axolotl PR #3510 analysis, "entropy and selective log-softmax
  with Triton kernels": section "Code analysis", part 1 (the per-row entropy
  of the softmax, ``entropy_from_logits``) and part 2
  (``selective_log_softmax`` forward and custom backward).

Where the pages leave a step open the plain reading is taken; each such
reading is named in the docstring of the function that takes it.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


# ---------------------------------------------------------------------------
# input decoding
# ---------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values.

    bf16 is the upper half of an IEEE binary32: the pattern shifted left by
    16 bits is the fp32 number it stands for, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(logits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return decode_bf16(logits)
    return np.asarray(logits, dtype=np.float64)


# ---------------------------------------------------------------------------
# softmax statistics, entropy, selective log-softmax
# ---------------------------------------------------------------------------
def log_softmax_stats(z: np.ndarray, temperature: float = 1.0):
    """u = z / T and the per-row log-sum-exp of u (two passes: max, then sum).

    Temperature divides the logits before the softmax [LIGER-BWD, "Code
    analysis": the gradient is divided by TEMPERATURE]."""
    u = np.asarray(z, dtype=np.float64) / np.float64(temperature)
    M = u.max(axis=1, keepdims=True)
    lse = M[:, 0] + np.log(np.exp(u - M).sum(axis=1))
    return u, lse


def selective_log_softmax(z: np.ndarray, index: np.ndarray, temperature: float = 1.0):
    """log_softmax(z / T)[r, index[r]] per row, and the row log-sum-exp.

    [AXOLOTL, "Code analysis" part 2: the log-softmax value of the logit at
    the given index of each row]."""
    u, lse = log_softmax_stats(z, temperature)
    r = np.arange(u.shape[0])
    return u[r, np.asarray(index, dtype=np.int64)] - lse, lse


def selective_log_softmax_bwd(z: np.ndarray, index: np.ndarray, grad_logp: np.ndarray,
                              temperature: float = 1.0) -> np.ndarray:
    """d/dz of sum_r grad_logp[r] * logp[r]: grad_r / T * (onehot(index_r) - softmax(z_r / T)).

    [AXOLOTL, "Code analysis" part 2: the custom backward of the selective
    log-softmax]; the softmax Jacobian is the textbook one."""
    u, lse = log_softmax_stats(z, temperature)
    p = np.exp(u - lse[:, None])
    onehot = np.zeros_like(p)
    onehot[np.arange(p.shape[0]), np.asarray(index, dtype=np.int64)] = 1.0
    g = np.asarray(grad_logp, dtype=np.float64)[:, None] / np.float64(temperature)
    return g * (onehot - p)


def entropy_from_logits(z: np.ndarray, temperature: float = 1.0):
    """Per-row entropy H = -sum_j p_j log p_j of p = softmax(z / T).

    [AXOLOTL, "Code analysis" part 1: the entropy of each row's softmax, from
    its log-softmax].  T is 1 in the page's op; a temperature divides the
    logits first, as in the GRPO path.  Written from the definition: the
    row's log-softmax log p = u - lse, then -sum exp(log p) log p."""
    u, lse = log_softmax_stats(z, temperature)
    logp = u - lse[:, None]
    return -(np.exp(logp) * logp).sum(axis=1)


# ---------------------------------------------------------------------------
# GRPO per-token terms
# ---------------------------------------------------------------------------
def ppo_clip_terms(x: np.ndarray, adv: np.ndarray, eps_low: float, eps_high: float):
    """PPO clipped-ratio surrogate per token, from the log-ratio x = logp - old_logp.

    ratio = e^x; clipped ratio = clip(ratio, 1 - eps_low, 1 + eps_high);
    pg = -min(ratio * A, clipped ratio * A).  The token counts as clipped when
    the clipped branch is strictly the smaller one (clipped * A < ratio * A);
    a clipped token carries no policy gradient [LIGER-BWD, "Why is this good":
    PPO-clipped tokens have dlogp = 0 when beta = 0].  Reading: closed clip
    interval, strict comparison for the flag (a tie keeps the gradient)."""
    ratio = np.exp(x)
    cr = np.clip(ratio, 1.0 - eps_low, 1.0 + eps_high)
    pg = -np.minimum(ratio * adv, cr * adv)
    is_clipped = cr * adv < ratio * adv
    return ratio, pg, is_clipped


def k3(d: np.ndarray) -> np.ndarray:
    """k3 KL estimator e^d - d - 1 with d = ref_logp - logp (written expm1(d) - d).

    Its derivative in logp is 1 - e^d, the KL gradient term of [LIGER-BWD,
    "Code analysis": BETA * (1 - exp(ref_logp - logp))]."""
    return np.expm1(d) - d


def _mask01(mask, n: int) -> np.ndarray:
    """Completion mask as float64 0/1: a nonzero entry is a kept token (the
    mask of a completion is 1 up to its length, 0 after it); None = all kept."""
    if mask is None:
        return np.ones(n)
    return (np.asarray(mask).reshape(-1) != 0).astype(np.float64)


def _advantage_per_row(adv, B, L):
    return np.repeat(np.asarray(adv, dtype=np.float64), L)


def grpo_forward(z, ids, old_logp, ref_logp, adv, mask, B, L, temperature, beta,
                 eps_low, eps_high, level="token"):
    """Forward row pass: lse, logp, entropy, kl and per-token loss.

    z: [B*L, V] (float values), row r = b*L + t.  ref_logp None means no
    reference model (ref == policy, kl == 0).  mask None means all ones.

    token level: loss = pg(x) + beta * k3(ref - logp), x = logp - old_logp.
    sequence level (reading; the page names only a "sequence level" backward
    whose KL term is scaled per token): x is averaged over the sequence's
    valid tokens, s_b = sum_t m x / max(sum_t m, 1); one ratio e^{s_b} per
    sequence; loss_bt = pg_b + beta * k3_bt.  The loss is reported for every
    token, masked or not; the mask enters through the caller's reduction."""
    z = np.asarray(z, dtype=np.float64)
    N = B * L
    assert z.shape[0] == N
    ids = np.asarray(ids, dtype=np.int64)
    logp, lse = selective_log_softmax(z, ids, temperature)
    H = entropy_from_logits(z, temperature)
    old = np.asarray(old_logp, dtype=np.float64)
    m = _mask01(mask, N)
    if ref_logp is None:
        d = np.zeros(N)
    else:
        d = np.asarray(ref_logp, dtype=np.float64) - logp
    kl = k3(d)
    kl_term = beta * kl if beta != 0.0 else np.zeros(N)
    A_row = _advantage_per_row(adv, B, L)
    out = dict(logp=logp, lse=lse, entropy=H, kl=kl,
               gathered=z[np.arange(N), ids].copy())
    if level == "token":
        ratio, pg, clipped = ppo_clip_terms(logp - old, A_row, eps_low, eps_high)
        out.update(loss=pg + kl_term, is_clipped=clipped, ratio=ratio)
    else:
        x = (logp - old).reshape(B, L)
        mm = m.reshape(B, L)
        n_b = np.maximum(mm.sum(axis=1), 1.0)
        s_b = (mm * x).sum(axis=1) / n_b
        ratio_b, pg_b, clipped_b = ppo_clip_terms(s_b, np.asarray(adv, np.float64),
                                                  eps_low, eps_high)
        out.update(loss=np.repeat(pg_b, L) + kl_term, is_clipped=np.repeat(clipped_b, L),
                   seq_ratio=ratio_b, seq_logratio=s_b, seq_n=n_b)
    return out


def grpo_dlogp(fwd: dict, ref_logp, adv, mask, dloss, B, L, beta, level="token"):
    """d(sum_r dloss_r * loss_r) / d logp_r per row (before the 1/T factor).

    token level [LIGER-BWD, "Code analysis", ``_grpo_loss_bwd_kernel``]:
      g = (-ratio * A * [not clipped] + beta * (1 - e^{ref - logp})) * dloss.
    sequence level [same section, ``_grpo_loss_bwd_kernel_seq``: KL term
    scaled by the token's own dloss]:
      g_bt = -ratio_b * A_b * [not clipped_b] * (sum_t' dloss_bt') * m_bt / n_b
             + beta * (1 - e^{ref - logp}) * dloss_bt."""
    N = B * L
    logp = fwd["logp"]
    w = np.asarray(dloss, dtype=np.float64)
    m = _mask01(mask, N)
    if ref_logp is None or beta == 0.0:
        kl_grad = np.zeros(N)
    else:
        kl_grad = beta * (1.0 - np.exp(np.asarray(ref_logp, np.float64) - logp))
    if level == "token":
        A_row = _advantage_per_row(adv, B, L)
        pg_grad = np.where(fwd["is_clipped"], 0.0, -fwd["ratio"] * A_row)
        return (pg_grad + kl_grad) * w
    A = np.asarray(adv, dtype=np.float64)
    clipped_b = fwd["is_clipped"].reshape(B, L)[:, 0]
    coef_b = np.where(clipped_b, 0.0, -fwd["seq_ratio"] * A)
    wsum_b = w.reshape(B, L).sum(axis=1)
    pg_grad = np.repeat(coef_b * wsum_b / fwd["seq_n"], L) * m
    return pg_grad + kl_grad * w


def dlogits_from_dlogp(z, ids, lse, g, temperature) -> np.ndarray:
    """dlogits_j = (g / T) * (1[j = y] - softmax(z / T)_j).

    Rows with g == 0 are exactly +0.0, the all-zero early path of [LIGER-BWD,
    "Code analysis": the added ``if dlogp == 0.0`` branch stores 0.0 over
    the row and returns]."""
    z = np.asarray(z, dtype=np.float64)
    u = z / np.float64(temperature)
    p = np.exp(u - np.asarray(lse, np.float64)[:, None])
    onehot = np.zeros_like(p)
    ids = np.asarray(ids, dtype=np.int64)
    onehot[np.arange(p.shape[0]), ids] = 1.0
    g = np.asarray(g, dtype=np.float64)
    dz = (g / np.float64(temperature))[:, None] * (onehot - p)
    dz[g == 0.0, :] = 0.0
    return dz


def grpo_backward(z, ids, old_logp, ref_logp, adv, mask, dloss, B, L, temperature, beta,
                  eps_low, eps_high, level="token", fwd: Optional[dict] = None):
    """dlogits of sum_r dloss_r * loss_r; returns (dz, g, zero_row)."""
    if fwd is None:
        fwd = grpo_forward(z, ids, old_logp, ref_logp, adv, mask, B, L, temperature,
                           beta, eps_low, eps_high, level)
    g = grpo_dlogp(fwd, ref_logp, adv, mask, dloss, B, L, beta, level)
    dz = dlogits_from_dlogp(z, ids, fwd["lse"], g, temperature)
    return dz, g, (g == 0.0)


# ---------------------------------------------------------------------------
# chunked fused-linear variant
# ---------------------------------------------------------------------------
def fused_linear_grpo(hidden, weight, ids, old_logp, ref_logp, adv, mask, dloss, B, L,
                      temperature, beta, eps_low, eps_high, chunk_seqs: int = 1):
    """Chunked LM-head + GRPO loss with gradients taken during the forward.

    [LIGER-TRL, detailed summary items 3-4]: the LM-head input is split along
    the batch; per chunk the logits h_c W^T are formed, the loss and its
    gradients for h_c and for W are computed at once, and the gradients are
    accumulated, so the full logits are never held.

    hidden [B*L, H], weight [V, H] (float values); returns
    (loss_sum = sum dloss * loss, grad_hidden [B*L, H], grad_weight [V, H])."""
    h = np.asarray(hidden, dtype=np.float64)
    W = np.asarray(weight, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    old = np.asarray(old_logp, dtype=np.float64)
    ref = None if ref_logp is None else np.asarray(ref_logp, dtype=np.float64)
    m = None if mask is None else np.asarray(mask)
    w = np.asarray(dloss, dtype=np.float64)
    adv = np.asarray(adv, dtype=np.float64)
    grad_h = np.zeros_like(h)
    grad_W = np.zeros_like(W)
    loss_sum = 0.0
    for b0 in range(0, B, chunk_seqs):
        nb = min(chunk_seqs, B - b0)
        rs = slice(b0 * L, (b0 + nb) * L)
        z = h[rs] @ W.T
        fwd = grpo_forward(z, ids[rs], old[rs], None if ref is None else ref[rs],
                           adv[b0:b0 + nb], None if m is None else m[rs], nb, L,
                           temperature, beta, eps_low, eps_high, "token")
        g = grpo_dlogp(fwd, None if ref is None else ref[rs], adv[b0:b0 + nb],
                       None if m is None else m[rs], w[rs], nb, L, beta, "token")
        dz = dlogits_from_dlogp(z, ids[rs], fwd["lse"], g, temperature)
        loss_sum += float((w[rs] * fwd["loss"]).sum())
        grad_h[rs] = dz @ W
        grad_W += dz.T @ h[rs]
    return loss_sum, grad_h, grad_W


def fused_linear_loss(hidden, weight, ids, old_logp, ref_logp, adv, mask, dloss, B, L,
                      temperature, beta, eps_low, eps_high) -> float:
    """sum dloss * loss of the unchunked composition (for finite differences)."""
    z = np.asarray(hidden, np.float64) @ np.asarray(weight, np.float64).T
    fwd = grpo_forward(z, ids, old_logp, ref_logp, adv, mask, B, L, temperature, beta,
                       eps_low, eps_high, "token")
    return float((np.asarray(dloss, np.float64) * fwd["loss"]).sum())


# ---------------------------------------------------------------------------
# steps either side of the row pass
# ---------------------------------------------------------------------------
def entropy_from_logits_bwd(z: np.ndarray, grad_entropy: np.ndarray,
                            temperature: float = 1.0) -> np.ndarray:
    """Gradient of sum_r g_r H_r with H_r the entropy of softmax(z_r / T)
    [AXOLOTL part 1 defines H = -sum p log p; the pages give it no backward].

    With u = z / T and log p = u - lse: dH/du_j = -p_j (log p_j + H), so
    dz_j = -(g / T) p_j (log p_j + H).  Written out from the definition with a
    two-pass softmax; rows with g = 0 get exact zeros."""
    u, lse = log_softmax_stats(z, temperature)
    logp = u - lse[:, None]
    p = np.exp(logp)
    H = -(p * logp).sum(axis=1)
    g = np.asarray(grad_entropy, dtype=np.float64)
    dz = -(g / np.float64(temperature))[:, None] * p * (logp + H[:, None])
    dz[g == 0.0] = 0.0
    return dz


def group_advantages(rewards: np.ndarray, group_size: int, eps: float = 1e-4,
                     scale: bool = True) -> np.ndarray:
    """Group-relative advantages of consecutive groups of `group_size`
    completions (one prompt each).

    The pages only name zero-advantage sequences [LIGER-BWD, summary]; they
    give no formula.  Reading (the plain meaning of "group-relative"): centre
    each group on its mean and, with `scale`, divide by the group's sample
    standard deviation (n - 1) plus eps.  A group whose rewards are all equal
    -- the zero-advantage case -- gets exactly 0 (the mean of equal floats can
    round away from them); a group of one has no spread and also gets 0."""
    r = np.asarray(rewards, dtype=np.float64).reshape(-1, group_size)
    out = np.zeros_like(r)
    for k in range(r.shape[0]):
        g = r[k]
        if g.max() == g.min():
            continue
        c = g - g.mean()
        out[k] = c / (g.std(ddof=1) + eps) if scale else c
    return out.reshape(-1)


def loss_weights(mask, B: int, L: int, reduction: str) -> np.ndarray:
    """Per-token upstream weights dloss = d(loss)/d(loss_bt) of a reduction
    of the per-token losses (NULL mask = all ones).

    The kernels take these weights as an input [LIGER-BWD "Code analysis":
    the backward scales by dloss]; the pages do not say which reduction.
    Readings: "token"     L = sum m l / max(sum m, 1)       (the harness's),
              "sequence"  L = (1/B) sum_b sum_t m l / max(n_b, 1),
              "constant"  L = sum m l / (B L)."""
    m = _mask01(mask, B * L).reshape(B, L)
    if reduction == "token":
        w = m / max(m.sum(), 1.0)
    elif reduction == "sequence":
        w = m / (np.maximum(m.sum(axis=1, keepdims=True), 1.0) * B)
    elif reduction == "constant":
        w = m / float(B * L)
    else:
        raise ValueError(reduction)
    return w.reshape(-1)
