"""Seeded synthetic inputs for the row-wise GRPO logits pass.

This module is shared by the float64 oracle side (tests) and the HIP side
(tests, bench, smoke).  It holds no arithmetic of the method itself: only
random draws, fp32 -> bf16 rounding of the draws, and the layout of the
arrays.  Quantities that need the policy's own log-probabilities (old_logp,
ref_logp = logp + noise) are returned as *noise* here; the caller adds the
true log-probabilities, which it takes from the oracle (tests) or from a
stored file written by the oracle (bench).  Likewise the per-token upstream
weights ``dloss`` of a loss reduction are not formed here: a case records
which reduction it stands for (``dloss_kind``: "mean" for the token mean,
"sum" for the plain sum) and leaves ``dloss`` to the caller, which takes it
from the oracle (tests) or from the library's ``grpo_loss_weights`` (bench).

Every draw comes from one ``numpy.random.SeedSequence(seed)`` split into the
named child streams of ``STREAMS`` (always in that order).  Large matrices are
drawn in fixed blocks of ``BLOCK_ROWS`` rows, block k from child k of its
stream, so any block can be regenerated on its own and the values do not
depend on the number of threads used.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

STREAMS = ("logits", "ids", "adv", "zero_choice", "old_noise", "ref_noise",
           "lengths", "peaks", "grad", "weight")
BLOCK_ROWS = 256

_POOL_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def streams(seed: int = 0) -> dict:
    kids = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return dict(zip(STREAMS, kids))


def _child(seq: np.random.SeedSequence, k: int) -> np.random.SeedSequence:
    # the k-th spawned child of ``seq``, built without mutating ``seq``
    return np.random.SeedSequence(entropy=seq.entropy,
                                  spawn_key=tuple(seq.spawn_key) + (k,))


# --------------------------------------------------------------------------
# dtype helpers (input encoding only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs must be finite (the generators never draw NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# blocked normal matrices
# --------------------------------------------------------------------------
def _fill_block(seq, k, n_cols, sigma, out_rows, bf16, peak_cols=None, peak=0.0,
                row0=0):
    g = np.random.default_rng(_child(seq, k))
    x = g.standard_normal((out_rows.shape[0], n_cols), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if peak_cols is not None:
        idx = np.arange(out_rows.shape[0])
        x[idx, peak_cols[row0:row0 + out_rows.shape[0]]] += np.float32(peak)
    out_rows[...] = f32_to_bf16_bits(x) if bf16 else x


def normal_matrix(seq: np.random.SeedSequence, n_rows: int, n_cols: int,
                  sigma: float, bf16: bool, peak_cols: Optional[np.ndarray] = None,
                  peak: float = 0.0, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """N(0, sigma^2) matrix drawn in BLOCK_ROWS-row blocks.

    ``peak_cols`` (one column per row) gets ``+peak`` before rounding.
    With ``rows`` given, only those rows are produced (same values as in the
    full matrix), in the order given."""
    dt = np.uint16 if bf16 else np.float32
    if rows is None:
        out = np.empty((n_rows, n_cols), dt)
        nb = (n_rows + BLOCK_ROWS - 1) // BLOCK_ROWS

        def job(k):
            r0 = k * BLOCK_ROWS
            r1 = min(n_rows, r0 + BLOCK_ROWS)
            _fill_block(seq, k, n_cols, sigma, out[r0:r1], bf16, peak_cols, peak, r0)

        with ThreadPoolExecutor(_POOL_THREADS) as ex:
            list(ex.map(job, range(nb)))
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, n_cols), dt)
    for blk in np.unique(rows // BLOCK_ROWS):
        r0 = int(blk) * BLOCK_ROWS
        r1 = min(n_rows, r0 + BLOCK_ROWS)
        tmp = np.empty((r1 - r0, n_cols), dt)
        _fill_block(seq, int(blk), n_cols, sigma, tmp, bf16, peak_cols, peak, r0)
        sel = np.nonzero(rows // BLOCK_ROWS == blk)[0]
        out[sel] = tmp[rows[sel] - r0]
    return out


# --------------------------------------------------------------------------
# GRPO row-pass cases
# --------------------------------------------------------------------------
@dataclasses.dataclass
class GrpoCase:
    """One GRPO logits-pass workload.

    logits: [N, V] fp32 values, or bf16 bits as uint16 (``dtype == "bf16"``).
    old_noise / ref_noise: the noise that the caller adds to the policy's own
    log-probabilities to form old_logp / ref_logp (ref_noise None: no
    reference model, ref == policy).  dloss is the per-token upstream weight
    (None until the caller fills it for the reduction named by dloss_kind).
    """
    name: str
    B: int
    L: int
    V: int
    dtype: str
    logits: Optional[np.ndarray]
    ids: np.ndarray
    adv: np.ndarray
    mask: np.ndarray
    old_noise: np.ndarray
    ref_noise: Optional[np.ndarray]
    dloss: Optional[np.ndarray]
    temperature: float
    beta: float
    eps_low: float
    eps_high: float
    level: str  # "token" | "sequence"
    seed: int = 0
    sigma: float = 2.0
    dloss_kind: str = "given"  # "mean" | "sum": dloss left to the caller

    @property
    def N(self) -> int:
        return self.B * self.L

    def logits_rows(self, rows) -> np.ndarray:
        """Regenerate only the given rows of the logits matrix."""
        s = streams(self.seed)
        return normal_matrix(s["logits"], self.N, self.V, self.sigma,
                             self.dtype == "bf16", rows=rows)


def _adv(s, B, zero_frac=None, zero_index=None):
    adv = np.random.default_rng(s["adv"]).standard_normal(B).astype(np.float32)
    if zero_index is not None:
        adv[zero_index] = 0.0
    if zero_frac is not None:
        nz = int(round(zero_frac * B))
        perm = np.random.default_rng(s["zero_choice"]).permutation(B)
        adv[perm[:nz]] = 0.0
    return adv


def _mask_from_lengths(s, B, L, lo, hi):
    lens = np.random.default_rng(s["lengths"]).integers(lo, hi + 1, size=B)
    t = np.arange(L)[None, :]
    return (t < lens[:, None]).astype(np.uint8).reshape(-1), lens


def _kind(dloss: str) -> str:
    if dloss not in ("mean", "sum"):
        raise ValueError(f"dloss reduction {dloss!r} (mean or sum)")
    return dloss


def tiny_case(variant: str = "a", seed: int = 0, with_logits: bool = True) -> GrpoCase:
    """B=2, L=16, V=1024, fp32 logits N(0, 2^2), T=1, eps 0.2/0.2, beta=0.04.

    variant "a": as stated; "b": beta=0; "c": no reference (ref == policy);
    "s": sequence-level loss; "t": as "a" with T=0.7 (exercises 1/T).
    dloss_kind "sum" (the parity tests' sum reduction, so dlogits is O(1))."""
    B, L, V = 2, 16, 1024
    s = streams(seed)
    z = normal_matrix(s["logits"], B * L, V, 2.0, bf16=False) if with_logits else None
    ids = np.random.default_rng(s["ids"]).integers(0, V, size=B * L).astype(np.int64)
    adv = _adv(s, B, zero_index=1)
    mask = np.ones(B * L, np.uint8)
    old_noise = (np.random.default_rng(s["old_noise"]).standard_normal(B * L) * 0.1).astype(np.float64)
    ref_noise = (np.random.default_rng(s["ref_noise"]).standard_normal(B * L) * 0.1).astype(np.float64)
    beta = 0.0 if variant == "b" else 0.04
    T = 0.7 if variant == "t" else 1.0
    return GrpoCase(name=f"tiny-{variant}", B=B, L=L, V=V, dtype="f32", logits=z, ids=ids,
                    adv=adv, mask=mask, old_noise=old_noise,
                    ref_noise=None if variant == "c" else ref_noise,
                    dloss=None, temperature=T, beta=beta,
                    eps_low=0.2, eps_high=0.2,
                    level="sequence" if variant == "s" else "token", seed=seed, sigma=2.0,
                    dloss_kind="sum")


def grpo_token_case(seed: int = 0, with_ref: bool = False, with_logits: bool = True,
                    B: int = 4, L: int = 512, V: int = 32000,
                    len_lo: Optional[int] = None, len_hi: Optional[int] = None,
                    dloss: str = "mean") -> GrpoCase:
    """Token-level GRPO workload: bf16 logits N(0, 2^2), T=0.9, beta=0.04,
    eps 0.2/0.28; half of the sequences have advantage exactly 0; old_logp
    noise N(0, 0.3^2) per token; trailing padding with lengths U{L/2..L}.

    At the default sizes (B=4, L=512, V=32000) this is the headline workload.
    ``with_ref`` False: no reference model (ref == policy, KL term identically
    0); True: ref noise N(0, 0.1^2).  ``dloss``: the reduction whose weights the
    caller supplies, "mean" (token mean) or "sum"."""
    s = streams(seed)
    N = B * L
    z = normal_matrix(s["logits"], N, V, 2.0, bf16=True) if with_logits else None
    ids = np.random.default_rng(s["ids"]).integers(0, V, size=N).astype(np.int64)
    adv = _adv(s, B, zero_frac=0.5)
    lo = L // 2 if len_lo is None else len_lo
    hi = L if len_hi is None else len_hi
    mask, _ = _mask_from_lengths(s, B, L, lo, hi)
    old_noise = np.random.default_rng(s["old_noise"]).standard_normal(N) * 0.3
    ref_noise = np.random.default_rng(s["ref_noise"]).standard_normal(N) * 0.1
    return GrpoCase(name=f"grpo-token-B{B}-L{L}-V{V}" + ("-ref" if with_ref else ""),
                    B=B, L=L, V=V, dtype="bf16", logits=z, ids=ids, adv=adv, mask=mask,
                    old_noise=old_noise, ref_noise=ref_noise if with_ref else None,
                    dloss=None, temperature=0.9, beta=0.04, eps_low=0.2, eps_high=0.28,
                    level="token", seed=seed, sigma=2.0, dloss_kind=_kind(dloss))


def grpo_sequence_case(seed: int = 0, with_logits: bool = True, B: int = 8, L: int = 1024,
                       V: int = 151936, dloss: str = "mean") -> GrpoCase:
    """Sequence-level GRPO workload with beta=0: bf16 logits N(0, 2^2), T=1,
    eps 0.2/0.28, a quarter of the advantages exactly 0, all-ones mask.
    The old_logp perturbation is one N(0, 0.5^2) draw per sequence, added to
    all of its tokens (so whole sequences fall outside the clip range)."""
    s = streams(seed)
    N = B * L
    z = normal_matrix(s["logits"], N, V, 2.0, bf16=True) if with_logits else None
    ids = np.random.default_rng(s["ids"]).integers(0, V, size=N).astype(np.int64)
    adv = _adv(s, B, zero_frac=0.25)
    mask = np.ones(N, np.uint8)
    delta = np.random.default_rng(s["old_noise"]).standard_normal(B) * 0.5
    old_noise = np.repeat(delta, L)
    return GrpoCase(name=f"grpo-seq-B{B}-L{L}-V{V}", B=B, L=L, V=V, dtype="bf16",
                    logits=z, ids=ids, adv=adv, mask=mask, old_noise=old_noise,
                    ref_noise=None, dloss=None, temperature=1.0, beta=0.0, eps_low=0.2,
                    eps_high=0.28, level="sequence", seed=seed, sigma=2.0,
                    dloss_kind=_kind(dloss))


@dataclasses.dataclass
class RowCase:
    """entropy_from_logits / selective_log_softmax workload (no loss)."""
    name: str
    N: int
    V: int
    logits: Optional[np.ndarray]  # bf16 bits [N, V]
    ids: np.ndarray
    grad: np.ndarray              # upstream grad of logp, fp32 [N]
    peak_cols: np.ndarray
    seed: int = 0
    sigma: float = 3.0
    peak: float = 8.0

    def logits_rows(self, rows) -> np.ndarray:
        s = streams(self.seed)
        return normal_matrix(s["logits"], self.N, self.V, self.sigma, True,
                             peak_cols=self.peak_cols, peak=self.peak, rows=rows)


def row_case(seed: int = 0, N: int = 65536, V: int = 32000, with_logits: bool = True) -> RowCase:
    """bf16 logits N(0, 3^2) with +8 added at one uniform column per row
    (independent of the sampled ids); ids uniform; upstream grad N(0, 1)."""
    s = streams(seed)
    peaks = np.random.default_rng(s["peaks"]).integers(0, V, size=N).astype(np.int64)
    z = (normal_matrix(s["logits"], N, V, 3.0, True, peak_cols=peaks, peak=8.0)
         if with_logits else None)
    ids = np.random.default_rng(s["ids"]).integers(0, V, size=N).astype(np.int64)
    grad = np.random.default_rng(s["grad"]).standard_normal(N).astype(np.float32)
    return RowCase(name=f"rows-N{N}-V{V}", N=N, V=V, logits=z, ids=ids, grad=grad,
                   peak_cols=peaks, seed=seed)


@dataclasses.dataclass
class FusedCase:
    """Chunked fused-linear GRPO workload: hidden [B*L, H] bf16 N(0,1),
    LM-head weight [V, H] bf16 N(0, 0.02^2), loss settings of the token-level
    workload (T=0.9, beta=0.04, eps 0.2/0.28, half the advantages 0, old noise
    N(0, 0.3^2), ref noise N(0, 0.1^2), lengths U{L/2..L})."""
    name: str
    B: int
    L: int
    H: int
    V: int
    hidden: Optional[np.ndarray]
    weight: Optional[np.ndarray]
    ids: np.ndarray
    adv: np.ndarray
    mask: np.ndarray
    old_noise: np.ndarray
    ref_noise: np.ndarray
    dloss: Optional[np.ndarray]
    temperature: float = 0.9
    beta: float = 0.04
    eps_low: float = 0.2
    eps_high: float = 0.28
    seed: int = 0
    w_sigma: float = 0.02
    dloss_kind: str = "given"

    @property
    def N(self) -> int:
        return self.B * self.L


def fused_case(seed: int = 0, B: int = 32, L: int = 1024, H: int = 1024, V: int = 151936,
               with_matrices: bool = True, dloss: str = "mean") -> FusedCase:
    s = streams(seed)
    N = B * L
    h = normal_matrix(s["logits"], N, H, 1.0, True) if with_matrices else None
    W = normal_matrix(s["weight"], V, H, 0.02, True) if with_matrices else None
    ids = np.random.default_rng(s["ids"]).integers(0, V, size=N).astype(np.int64)
    adv = _adv(s, B, zero_frac=0.5)
    mask, _ = _mask_from_lengths(s, B, L, L // 2, L)
    old_noise = np.random.default_rng(s["old_noise"]).standard_normal(N) * 0.3
    ref_noise = np.random.default_rng(s["ref_noise"]).standard_normal(N) * 0.1
    return FusedCase(name=f"fused-B{B}-L{L}-H{H}-V{V}", B=B, L=L, H=H, V=V, hidden=h,
                     weight=W, ids=ids, adv=adv, mask=mask, old_noise=old_noise,
                     ref_noise=ref_noise, dloss=None, seed=seed, dloss_kind=_kind(dloss))


def add_noise_f32(logp_true: np.ndarray, noise: np.ndarray) -> np.ndarray:
    """old/ref log-probabilities: true policy logp plus noise, stored as fp32."""
    return (np.asarray(logp_true, np.float64) + np.asarray(noise, np.float64)).astype(np.float32)


# --------------------------------------------------------------------------
# stored policy log-probabilities (written by tests/golden/make_oracle_logp.py)
# --------------------------------------------------------------------------
_GOLDEN = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "tests", "golden")


def load_stored_logp(name: str, check_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """float64 [B*L] policy logp of the named workload ("token", "sequence",
    "fused").  ``check_rows``: the generator's bits for the stored check rows,
    compared against the stored digest (raises if the inputs have drifted)."""
    import hashlib
    import json
    with open(os.path.join(_GOLDEN, f"oracle_logp_{name}.json")) as f:
        meta = json.load(f)
    if check_rows is not None:
        d = hashlib.sha256(np.ascontiguousarray(check_rows).tobytes()).hexdigest()
        if not meta["check_digest"].startswith(d):
            raise RuntimeError(f"stored logp '{name}' does not match the generated inputs")
    return np.load(os.path.join(_GOLDEN, f"oracle_logp_{name}.npy"))


def stored_check_rows(name: str):
    import json
    with open(os.path.join(_GOLDEN, f"oracle_logp_{name}.json")) as f:
        return json.load(f)["check_rows"]


def load_stored_lse(name: str) -> np.ndarray:
    """float64 [B*L] row log-sum-exp stored beside ``load_stored_logp``."""
    return np.load(os.path.join(_GOLDEN, f"oracle_lse_{name}.npy"))
