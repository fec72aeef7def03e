"""A seeded sweep of the GRPO row path (two-pass and, at token level, the
single pass) across the boundaries where the kernels change shape: row
lengths of 1 to 8193 16-byte vectors with and without a tail (the single
pass's one-wave, 256-, 1024- and 512-lane shapes, the backward's 512- and
4096-vector chunks, the two-pass fallback past 8192 vectors), 16-byte and
odd row pitches, both levels, both dtypes, temperatures around 1, with and
without a reference model, zero advantages and masked tokens.  Each case is
checked against the oracle with the bars of test_rows_gpu."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import GrpoInputs, logits_to_dev, require_gpu, run_grpo_gpu, say
from test_fused_rows_gpu import run_single_pass
from test_rows_gpu import check_backward, check_forward, oracle_expectations

pytestmark = pytest.mark.gpu

NVEC = [1, 63, 64, 255, 256, 257, 511, 512, 513, 2047, 2048, 2049, 4095, 4096, 4097, 8191,
        8192, 8193]


def _case(k):
    rng = np.random.default_rng(1000 + k)
    dtype = "f32" if k % 2 == 0 else "bf16"
    es = 4 if dtype == "f32" else 2
    VE = 16 // es
    V = int(NVEC[k % len(NVEC)] * VE + rng.choice([0, 1, VE - 1]))
    aligned_pad = (-V) % VE
    ld_extra = int(rng.choice([aligned_pad, aligned_pad + VE, 1 if aligned_pad != 1 else 3]))
    level = "sequence" if k % 4 >= 2 else "token"
    B, L = int(rng.choice([1, 2, 3])), int(rng.choice([1, 2, 5]))
    T = float(rng.choice([0.6, 1.0, 1.4]))
    beta = float(rng.choice([0.0, 0.04]))
    with_ref = beta > 0 or bool(rng.integers(2))
    zf = (rng.standard_normal((B * L, V + ld_extra)) * 2.0).astype(np.float32)
    zb = synth.f32_to_bf16_bits(zf) if dtype == "bf16" else zf
    z64 = oracle.to_f64(zb, dtype)[:, :V]
    ids = rng.integers(0, V, B * L).astype(np.int64)
    adv = rng.standard_normal(B).astype(np.float32)
    adv[rng.integers(B)] = 0.0 if B > 1 else adv[0]
    mask = (rng.random(B * L) < 0.8).astype(np.uint8)
    mask[::L] = 1  # every sequence keeps a token
    dloss = (mask * rng.uniform(0.5, 1.5, B * L)).astype(np.float32)
    lp, _ = oracle.selective_log_softmax(z64, ids, T)
    case = synth.GrpoCase(name=f"sweep-{k}", B=B, L=L, V=V, dtype=dtype, logits=None, ids=ids,
                          adv=adv, mask=mask, old_noise=rng.standard_normal(B * L) * 0.3,
                          ref_noise=rng.standard_normal(B * L) * 0.1 if with_ref else None,
                          dloss=dloss, temperature=T, beta=beta, eps_low=0.2, eps_high=0.28,
                          level=level)
    return case, zb, z64, ld_extra


@pytest.mark.parametrize("k", range(36))
def test_row_path_sweep(k):
    lib = require_gpu()
    case, zb, z64, ld_extra = _case(k)
    say(f"sweep {k}: {case.dtype} V={case.V} ld=V+{ld_extra} {case.level} B={case.B} "
        f"L={case.L} T={case.temperature} beta={case.beta} ref={case.ref_noise is not None}")
    t = logits_to_dev(zb, case.dtype)[:, :case.V]
    inp = GrpoInputs(case, oracle.selective_log_softmax(z64, case.ids, case.temperature)[0])
    fwd, dz, zr = run_grpo_gpu(lib, t, inp)
    o, g = oracle_expectations(inp, z64, fwd)
    check_forward(case, o, fwd, ref=inp.ref)
    check_backward(case, o, g, dz, zr, z64, inp)
    if case.level == "token":
        one, dz1, zr1 = run_single_pass(lib, t, inp)
        o1, g1 = oracle_expectations(inp, z64, one)
        check_forward(case, o1, one, ref=inp.ref)
        check_backward(case, o1, g1, dz1, zr1, z64, inp)


@pytest.mark.parametrize("k", range(24))
def test_entropy_selective_sweep(k):
    """entropy_from_logits, selective_log_softmax and its backward, and the
    entropy backward over the same row-length and pitch boundaries.  The
    backwards take the oracle's lse and H rounded to fp32.  Bars: the
    forwards as in test_rows_gpu; the selective backward in fp32 within
    2^-21 |g/T| p (1 + |z|/T + |lse|) + 2^-22 |o| (the exponent's and the
    product's fp32 roundings, the inputs' rounding included), in bf16 the
    output rounding's bar; the entropy backward as in test_aux_gpu."""
    from test_aux_gpu import _entropy_bound
    from gpu_common import assert_bf16_dz, assert_rel, bits, dev, dev_to_f64
    import torch
    lib = require_gpu()
    rng = np.random.default_rng(2000 + k)
    dtype = "f32" if k % 2 == 0 else "bf16"
    es = 4 if dtype == "f32" else 2
    VE = 16 // es
    V = int(NVEC[(5 * k) % len(NVEC)] * VE + rng.choice([0, 1, VE - 1]))
    aligned_pad = (-V) % VE
    ld_extra = int(rng.choice([aligned_pad, aligned_pad + VE, 1 if aligned_pad != 1 else 3]))
    N = int(rng.integers(1, 13))
    T = float(rng.choice([0.6, 1.0, 1.4]))
    say(f"entropy/selective sweep {k}: {dtype} V={V} ld=V+{ld_extra} N={N} T={T}")
    zf = (rng.standard_normal((N, V + ld_extra)) * 3.0).astype(np.float32)
    zb = synth.f32_to_bf16_bits(zf) if dtype == "bf16" else zf
    t = logits_to_dev(zb, dtype)[:, :V]
    z64 = oracle.to_f64(zb, dtype)[:, :V]
    ids = rng.integers(0, V, N).astype(np.int64)
    g = rng.standard_normal(N).astype(np.float32)
    g[rng.integers(N)] = 0.0
    H = lib.entropy_from_logits(t, temperature=T)
    logp, lse = lib.selective_log_softmax(t, dev(ids), temperature=T)
    _, lse_o = oracle.log_softmax_stats(z64, T)
    H_o = oracle.entropy_from_logits(z64, T)
    lp_o, _ = oracle.selective_log_softmax(z64, ids, T)
    lse32, H32 = lse_o.astype(np.float32), H_o.astype(np.float32)
    dz = lib.selective_log_softmax_bwd(t, dev(ids), dev(lse32), dev(g), temperature=T)
    dzH = lib.entropy_from_logits_bwd(t, dev(lse32), dev(H32), dev(g), temperature=T)
    torch.cuda.synchronize()
    assert_rel(H.cpu().numpy(), H_o, "entropy")
    assert_rel(logp.cpu().numpy(), lp_o, "logp")
    assert_rel(lse.cpu().numpy(), lse_o, "lse")
    want = oracle.selective_log_softmax_bwd(z64, ids, g.astype(np.float64), T)
    got = dev_to_f64(dz)
    if dtype == "bf16":
        assert_bf16_dz(got, want)
    else:
        p = np.exp(z64 / T - lse_o[:, None])
        tol = (np.abs(g.astype(np.float64)) / T)[:, None] * p * 2.0 ** -21 * (
            1 + np.abs(z64) / T + np.abs(lse_o)[:, None]) + 2.0 ** -22 * np.abs(want) + 1e-30
        assert (np.abs(got - want) <= tol).all(), np.abs(got - want).max()
    assert (bits(dz)[g == 0.0] == 0).all()
    wantH = oracle.entropy_from_logits_bwd(z64, g.astype(np.float64), T)
    tolH = 1e-5 * np.abs(wantH) + _entropy_bound(z64, T, g, lse_o, H_o) + 1e-30
    if dtype == "bf16":
        tolH = tolH + 2.0 ** -8 * np.abs(wantH)
    errH = np.abs(dev_to_f64(dzH) - wantH)
    assert (errH <= tolH).all(), errH.max()
    assert (bits(dzH)[g == 0.0] == 0).all()
