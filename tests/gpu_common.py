"""Helpers shared by the GPU parity tests (device tensors, comparisons, runners)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

# per-row fp32 outputs (loss, logp, lse, entropy, kl): 1e-5 relative with an
# absolute floor for values near zero
RTOL, ATOL = 1e-5, 1e-6
BF16_DZ_ATOL = 2e-2


def bf16_dz_tol(want) -> np.ndarray:
    """Per-element bar for bf16 dlogits: 2e-2 absolute, or one bf16 ulp of the
    oracle's value where that is larger (|o| >= 4, where the spacing of bf16
    numbers is 2^-5 or more, so even the correctly rounded value can sit
    more than 2e-2 from the exact one; half an ulp is the rounding, the other
    half the kernel's fp32 arithmetic before it)."""
    a = np.abs(np.asarray(want, np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.where(a > 0, np.exp2(e - 7), 0.0)
    return np.maximum(BF16_DZ_ATOL, ulp)


def assert_bf16_dz(got, want, name="bf16 dlogits"):
    err = np.abs(np.asarray(got, np.float64) - want)
    tol = bf16_dz_tol(want)
    bad = ~(err <= tol)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError(f"{name}: {bad.sum()} elements over the bar; max err {err.max()}; "
                             f"got {np.asarray(got).ravel()[i].tolist()} want {want.ravel()[i].tolist()}")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import rl_fine_tuning_row_amd as lib
    lib.lib()  # raises if the HIP library is not built
    return lib


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def logits_to_dev(z: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(z).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)).cuda()


def dev_to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.decode_bf16(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy().view(np.uint32)


def assert_rel(got, want, name, rtol=RTOL, atol=ATOL, where=None):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    tol = rtol * np.abs(want) + atol
    bad = ~(err <= tol)
    if where is not None:
        bad &= where
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} outside |d| <= {rtol}*|o| + {atol}; "
                             f"idx {i.tolist()} got {got.ravel()[i].tolist()} want {want.ravel()[i].tolist()}")
    return float((err / (np.abs(want) + atol)).max()) if err.size else 0.0


def kink_distance(x, eps_low, eps_high):
    lo, hi = np.log1p(-eps_low), np.log1p(eps_high)
    return np.minimum(np.abs(x - lo), np.abs(x - hi))


class GrpoInputs:
    """Host (numpy) inputs of one GRPO case with old/ref log-probabilities."""

    def __init__(self, case: synth.GrpoCase, logp_true: np.ndarray):
        self.case = case
        self.old = synth.add_noise_f32(logp_true, case.old_noise)
        self.ref = None if case.ref_noise is None else synth.add_noise_f32(logp_true, case.ref_noise)

    def oracle_args(self, z64, rows=None):
        c = self.case
        return dict(z=z64, ids=c.ids, old_logp=self.old.astype(np.float64),
                    ref_logp=None if self.ref is None else self.ref.astype(np.float64),
                    adv=c.adv, mask=c.mask, B=c.B, L=c.L, temperature=c.temperature,
                    beta=c.beta, eps_low=c.eps_low, eps_high=c.eps_high, level=c.level)

    def to_dev(self):
        c = self.case
        d = dict(ids=dev(c.ids), old_logp=dev(self.old), adv=dev(c.adv), mask=dev(c.mask),
                 dloss=dev(c.dloss),
                 ref_logp=None if self.ref is None else dev(self.ref))
        return d


def run_grpo_gpu(lib, logits_t, inp: GrpoInputs, d=None, force_dense=False, dloss=None,
                 gathered=True):
    c = inp.case
    d = d or inp.to_dev()
    kw = dict(temperature=c.temperature, beta=c.beta, eps_low=c.eps_low, eps_high=c.eps_high,
              level=c.level)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fwd = lib.grpo_logits_fwd(logits_t, d["ids"], d["old_logp"], d["adv"], c.B, c.L,
                              ref_logp=d["ref_logp"], mask=d["mask"], gathered=gathered,
                              err_count=err, **kw)
    dz, zr = lib.grpo_logits_bwd(logits_t, d["ids"], d["old_logp"], d["adv"], c.B, c.L,
                                 fwd["logp"], fwd["lse"], d["dloss"] if dloss is None else dloss,
                                 ref_logp=d["ref_logp"], mask=d["mask"],
                                 seq_ratio=fwd.get("seq_ratio"), force_dense=force_dense, **kw)
    torch.cuda.synchronize()
    fwd["err_count"] = err
    return fwd, dz, zr
