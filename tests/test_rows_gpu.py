"""GPU parity of the row kernels against the float64 oracle (through the C ABI).

Tolerances:
  * fp32 per-row outputs (loss, logp, lse, entropy, kl, seq_ratio):
    |gpu - oracle| <= 1e-5 |oracle| + 1e-6;
  * gathered logits, zero_row, err_count: bit-exact;
  * is_clipped: exact, except where the oracle's log-ratio lies within the
    forward tolerance of a clip boundary (there the row is compared against
    the branch the GPU took);
  * bf16 dlogits: 2e-2 absolute, or one bf16 ulp of the oracle value where
    that is larger (|o| >= 4, reached with sum-reduction weights at low
    temperature: |g/T| = 20 at T = 0.05);
  * fp32 dlogits: the forward tolerance carried through the backward formula.
    With e_logp = 1e-5|logp| + 1e-6 and e_lse = 1e-5|lse| + 1e-6 (the bounds
    the forward meets), the row coefficient g/T moves by at most
    (|ratio A| [not clipped] + beta e^{ref - logp}) |dloss| / T * e_logp
    (the derivative of dlogp in logp, times the logp error; at sequence level
    the ratio term carries the sequence's mean error), and
    p_j = e^{u_j - lse} by p_j e_lse, so
    |d dz_j| <= that + |g/T| (e_lse + 1e-6);
  * rows with dlogp == 0: exactly +0.0.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from case_weights import fill_dloss
from gpu_common import (GrpoInputs, assert_bf16_dz, assert_rel, bits, dev, dev_to_f64,
                        kink_distance, logits_to_dev, require_gpu, run_grpo_gpu, say)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# shared checker
# ---------------------------------------------------------------------------
def oracle_expectations(inp: GrpoInputs, z64, fwd_gpu, logp_all=None):
    """Oracle forward and dlogp, with is_clipped taken from the GPU only where
    the oracle's log-ratio is within the forward tolerance of a clip kink."""
    c = inp.case
    args = inp.oracle_args(z64)
    o = oracle.grpo_forward(**args)
    gpu_clip = fwd_gpu["is_clipped"].cpu().numpy().astype(bool)
    if c.level == "token":
        x = o["logp"] - inp.old
        near = kink_distance(x, c.eps_low, c.eps_high) < 1e-5 * (1 + np.abs(o["logp"])) + 1e-6
    else:
        xb = o["seq_logratio"]
        near = np.repeat(kink_distance(xb, c.eps_low, c.eps_high) < 2e-5 * (1 + np.abs(xb)), c.L)
    mism = gpu_clip != o["is_clipped"]
    assert not (mism & ~near).any(), f"is_clipped differs away from a clip boundary: {np.flatnonzero(mism & ~near)[:8]}"
    if mism.any():
        say(f"  {mism.sum()} is_clipped flags differ within the boundary tolerance; using the GPU branch there")
        o["is_clipped"] = np.where(mism, gpu_clip, o["is_clipped"])
    g = oracle.grpo_dlogp(o, args["ref_logp"], c.adv, c.mask, c.dloss, c.B, c.L, c.beta, c.level)
    return o, g


def logp_slopes(c, o, ref):
    """|d kl / d logp| and |d loss / d logp| per row, and the logp error bar
    e_logp = 1e-5 |logp| + 1e-6 they carry into kl and the loss (module doc):
    kl = e^d - d - 1 with d = ref - logp moves by |e^d - 1| e_logp; the loss
    by |ratio A| [not clipped] e_logp + beta |e^d - 1| e_logp (at sequence
    level the ratio term takes the largest e_logp of the sequence, the bar of
    its mean log-ratio)."""
    logp = o["logp"]
    e = 1e-5 * np.abs(logp) + 1e-6
    kl_s = np.abs(np.expm1(ref - logp)) if ref is not None else np.zeros_like(logp)
    A = np.abs(np.repeat(np.asarray(c.adv, np.float64), c.L))
    if c.level == "token":
        pg = np.where(o["is_clipped"], 0.0, o["ratio"] * A) * e
    else:
        e_seq = np.repeat(e.reshape(c.B, c.L).max(1), c.L)
        pg = np.where(o["is_clipped"], 0.0, np.repeat(o["seq_ratio"], c.L) * A) * e_seq
    return kl_s * e, pg + c.beta * kl_s * e


def check_forward(c, o, fwd, logits_bits=None, ref=None):
    """Per-row outputs against the oracle: logp, lse, entropy at 1e-5 |o| + 1e-6;
    kl and the loss, computed from logp, also within what logp's own bar
    carries into them (logp_slopes)."""
    assert_rel(fwd["logp"].cpu().numpy(), o["logp"], "logp")
    assert_rel(fwd["lse"].cpu().numpy(), o["lse"], "lse")
    assert_rel(fwd["entropy"].cpu().numpy(), o["entropy"], "entropy")
    e_kl, e_loss = logp_slopes(c, o, ref)
    assert_rel(fwd["kl"].cpu().numpy(), o["kl"], "kl", atol=1e-6 + e_kl)
    assert_rel(fwd["loss"].cpu().numpy(), o["loss"], "loss", atol=1e-6 + e_loss)
    if fwd.get("gathered") is not None:
        g = fwd["gathered"].cpu().numpy()
        assert np.array_equal(g.astype(np.float64), o["gathered"]), "gathered not bit-exact"
    if c.level == "sequence":
        assert_rel(fwd["seq_ratio"].cpu().numpy(), o["seq_ratio"], "seq_ratio")
    assert int(fwd["err_count"].item()) == 0


def coef_error_bound(c, inp, o, logp):
    """Bound on |d(g/T)| from the forward's logp tolerance (see module doc)."""
    e_logp = 1e-5 * np.abs(logp) + 1e-6
    w = np.abs(c.dloss.astype(np.float64))
    A = np.abs(np.repeat(c.adv.astype(np.float64), c.L))
    clipped = o["is_clipped"]
    if c.level == "token":
        pg = np.where(clipped, 0.0, np.exp(logp - inp.old) * A) * w
    else:
        e_seq = np.repeat(e_logp.reshape(c.B, c.L).max(1), c.L)
        wsum = np.repeat(w.reshape(c.B, c.L).sum(1), c.L)
        m = c.mask.astype(np.float64)
        ratio = np.repeat(o["seq_ratio"], c.L)
        pg = np.where(clipped, 0.0, ratio * A) * wsum * m / np.repeat(o["seq_n"], c.L)
        e_logp = np.maximum(e_logp, e_seq)
    kl = 0.0
    if inp.ref is not None and c.beta != 0.0:
        kl = c.beta * np.exp(inp.ref.astype(np.float64) - logp) * w
    return (pg + kl) * e_logp / c.temperature


def check_backward(c, o, g, dz, zr, z64, inp):
    zero_exp = g == 0.0
    zr = zr.cpu().numpy().astype(bool)
    assert np.array_equal(zr, zero_exp), f"zero_row differs at {np.flatnonzero(zr != zero_exp)[:8]}"
    dz_o = oracle.dlogits_from_dlogp(z64, c.ids, o["lse"], g, c.temperature)
    got = dev_to_f64(dz)
    # zero rows are exactly +0.0 (sign bit clear)
    b = bits(dz)
    assert (b[zero_exp] == 0).all(), "zero rows are not +0.0"
    coef = g / c.temperature
    if dz.dtype == torch.bfloat16:
        assert_bf16_dz(got, dz_o)
    else:
        tol = coef_error_bound(c, inp, o, o["logp"]) + np.abs(coef) * (1e-5 * np.abs(o["lse"]) + 2e-6)
        err = np.abs(got - dz_o)
        bad = err > tol[:, None]
        assert not bad.any(), f"fp32 dlogits: {bad.sum()} elements over tolerance, max err {err.max()}"
    rs = np.abs(got.sum(axis=1))
    assert (rs <= 1e-2 * np.abs(coef) + 1e-6).all(), f"row sums {rs.max()}"


def _tiny(variant):
    case = fill_dloss(synth.tiny_case(variant))
    z64 = case.logits.astype(np.float64)
    logp_true, _ = oracle.selective_log_softmax(z64, case.ids, case.temperature)
    return case, z64, GrpoInputs(case, logp_true)


# ---------------------------------------------------------------------------
# tiny GRPO case: B=2, L=16, V=1024, fp32
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["a", "b", "c", "s", "t"])
def test_tiny_grpo_parity(variant):
    lib = require_gpu()
    case, z64, inp = _tiny(variant)
    say(f"tiny GRPO parity: variant {variant}, B={case.B} L={case.L} V={case.V} fp32, seed 0")
    fwd, dz, zr = run_grpo_gpu(lib, logits_to_dev(case.logits, "f32"), inp)
    o, g = oracle_expectations(inp, z64, fwd)
    check_forward(case, o, fwd, ref=inp.ref)
    check_backward(case, o, g, dz, zr, z64, inp)
    if variant in ("b", "c"):
        # zero-advantage sequence: exactly zero rows
        assert zr.cpu().numpy()[case.L:].all()


@pytest.mark.parametrize("variant", ["a", "b", "c", "s"])
def test_tiny_skip_equals_dense(variant):
    """The early all-zero path gives the same dlogits as the dense path
    (bitwise up to the sign of zero, the torch.equal criterion)."""
    lib = require_gpu()
    case, z64, inp = _tiny(variant)
    say(f"tiny skip-vs-dense: variant {variant}")
    t = logits_to_dev(case.logits, "f32")
    _, dz1, zr1 = run_grpo_gpu(lib, t, inp)
    _, dz2, zr2 = run_grpo_gpu(lib, t, inp, force_dense=True)
    assert torch.equal(dz1, dz2) and torch.equal(zr1, zr2)


# ---------------------------------------------------------------------------
# headline token-level case: B=4, L=512, V=32000, bf16
# ---------------------------------------------------------------------------
def _token_case(with_ref, dloss):
    case = fill_dloss(synth.grpo_token_case(with_ref=with_ref, dloss=dloss))
    logp = synth.load_stored_logp("token", case.logits[synth.stored_check_rows("token")])
    return case, GrpoInputs(case, logp)


@pytest.mark.parametrize("with_ref", [False, True])
@pytest.mark.parametrize("dloss", ["sum", "mean"])
def test_token_level_parity(with_ref, dloss):
    lib = require_gpu()
    case, inp = _token_case(with_ref, dloss)
    say(f"token-level GRPO parity: B4 L512 V32000 bf16, ref={'noise' if with_ref else 'policy'}, dloss={dloss}")
    t = logits_to_dev(case.logits, "bf16")
    fwd, dz, zr = run_grpo_gpu(lib, t, inp)
    z64 = oracle.decode_bf16(case.logits)
    o, g = oracle_expectations(inp, z64, fwd)
    check_forward(case, o, fwd, ref=inp.ref)
    check_backward(case, o, g, dz, zr, z64, inp)
    say(f"  zero rows: {int(zr.sum())} of {case.N}; clipped: {int(fwd['is_clipped'].sum())}")
    # skip vs forced dense on the same inputs
    _, dz2, zr2 = run_grpo_gpu(lib, t, inp, force_dense=True)
    assert torch.equal(dz, dz2) and torch.equal(zr, zr2)


def test_token_level_deterministic_and_guarded():
    """Two runs are bitwise equal; guard rows around the output stay untouched."""
    lib = require_gpu()
    case, inp = _token_case(False, "sum")
    say("token-level determinism + guard bands")
    t = logits_to_dev(case.logits, "bf16")
    fwd, dz, zr = run_grpo_gpu(lib, t, inp)
    fwd2, dz2, zr2 = run_grpo_gpu(lib, t, inp)
    for k in ("loss", "logp", "lse", "entropy", "kl", "is_clipped"):
        assert torch.equal(fwd[k], fwd2[k]), k
    assert torch.equal(bits_t(dz), bits_t(dz2))
    d = inp.to_dev()
    guard = torch.full((case.N + 4, case.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    sentinel = guard.view(torch.int16).clone()
    out = guard[2:2 + case.N]
    lib.grpo_logits_bwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L, fwd["logp"],
                        fwd["lse"], d["dloss"], mask=d["mask"], temperature=case.temperature,
                        beta=case.beta, eps_low=case.eps_low, eps_high=case.eps_high,
                        dlogits=out)
    torch.cuda.synchronize()
    gv = guard.view(torch.int16)
    assert torch.equal(gv[:2], sentinel[:2]) and torch.equal(gv[-2:], sentinel[-2:])
    assert torch.equal(out.view(torch.int16), dz.view(torch.int16))


def bits_t(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_token_level_inputs_unchanged_and_row_outputs_guarded():
    """No call writes to its inputs (logits, ids, old_logp, ref_logp, adv,
    mask, dloss, and the backward's logp / lse stay bit-identical), and the
    per-row outputs of the forward, the backward and the single pass write
    exactly their B*L entries: NaN guard bands of 64 entries on either side
    of every output buffer stay untouched."""
    lib = require_gpu()
    case, inp = _token_case(True, "sum")
    say("token-level canaries: inputs bit-unchanged, guard bands around per-row outputs")
    t = logits_to_dev(case.logits, "bf16")
    d = inp.to_dev()
    N, G = case.N, 64
    kw = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
              eps_high=case.eps_high)

    def guarded(dtype):
        # the returned full buffer is the bit view the guards are compared on
        # (NaN != NaN for torch.equal on floats)
        if dtype == torch.float32:
            full = torch.full((N + 2 * G,), float("nan"), dtype=dtype, device="cuda")
            return full.view(torch.int32), full[G:G + N]
        full = torch.full((N + 2 * G,), 0xA5, dtype=dtype, device="cuda")
        return full, full[G:G + N]

    def snap(ts):
        return [x.clone() for x in ts]

    inputs = [t.view(torch.int16), d["ids"], d["old_logp"], d["ref_logp"], d["adv"], d["mask"],
              d["dloss"]]
    before = snap(inputs)
    fulls, out = {}, {}
    for k in ("loss", "logp", "lse", "entropy", "kl", "gathered"):
        fulls[k], out[k] = guarded(torch.float32)
    fulls["is_clipped"], out["is_clipped"] = guarded(torch.uint8)
    guards = {k: (v[:G].clone(), v[G + N:].clone()) for k, v in fulls.items()}
    fwd = lib.grpo_logits_fwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L,
                              ref_logp=d["ref_logp"], mask=d["mask"], out=out, gathered=True, **kw)
    logp_lse = snap([fwd["logp"], fwd["lse"]])
    zfull, zr = guarded(torch.uint8)
    zguard = (zfull[:G].clone(), zfull[G + N:].clone())
    lib.grpo_logits_bwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L, fwd["logp"],
                        fwd["lse"], d["dloss"], ref_logp=d["ref_logp"], mask=d["mask"],
                        zero_row=zr, **kw)
    torch.cuda.synchronize()
    for a, b in zip(inputs + [fwd["logp"], fwd["lse"]], before + logp_lse):
        assert torch.equal(a, b)
    # the single pass into fresh guarded buffers
    fulls1, out1 = {}, {}
    for k in ("loss", "logp", "lse", "entropy", "kl"):
        fulls1[k], out1[k] = guarded(torch.float32)
    fulls1["is_clipped"], out1["is_clipped"] = guarded(torch.uint8)
    guards1 = {k: (v[:G].clone(), v[G + N:].clone()) for k, v in fulls1.items()}
    z1full, zr1 = guarded(torch.uint8)
    z1guard = (z1full[:G].clone(), z1full[G + N:].clone())
    lib.grpo_logits_fwd_bwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L, d["dloss"],
                            ref_logp=d["ref_logp"], mask=d["mask"], out=out1, zero_row=zr1, **kw)
    torch.cuda.synchronize()
    for a, b in zip(inputs, before):
        assert torch.equal(a, b)
    for fs, gs in ((fulls, guards), (fulls1, guards1)):
        for k, v in fs.items():
            lo, hi = gs[k]
            assert torch.equal(v[:G], lo) and torch.equal(v[G + N:], hi), f"{k} guard band written"
    for full, (lo, hi) in ((zfull, zguard), (z1full, z1guard)):
        assert torch.equal(full[:G], lo) and torch.equal(full[G + N:], hi), "zero_row guard band"
    # the guarded outputs hold the same values as unguarded runs
    ref_fwd, _, ref_zr = run_grpo_gpu(lib, t, inp)
    for k in ("loss", "logp", "lse", "entropy", "kl", "is_clipped"):
        assert torch.equal(out[k], ref_fwd[k]), k
    assert torch.equal(zr, ref_zr) and torch.equal(zr1, ref_zr)


# ---------------------------------------------------------------------------
# sequence-level case: B=8, L=1024, V=151936, bf16, beta = 0
# ---------------------------------------------------------------------------
def test_sequence_level_parity():
    lib = require_gpu()
    case = fill_dloss(synth.grpo_sequence_case(dloss="sum"))
    logp_true = synth.load_stored_logp("sequence", case.logits[synth.stored_check_rows("sequence")])
    inp = GrpoInputs(case, logp_true)
    say("sequence-level GRPO parity: B8 L1024 V151936 bf16, beta 0")
    t = logits_to_dev(case.logits, "bf16")
    fwd, dz, zr = run_grpo_gpu(lib, t, inp)
    # every row: logp against the stored oracle logp; sequence quantities and
    # dlogp from the oracle's definitions on that logp
    assert_rel(fwd["logp"].cpu().numpy(), logp_true, "logp (all rows)")
    o = dict(logp=logp_true)
    x = (logp_true - inp.old).reshape(case.B, case.L)
    m = case.mask.reshape(case.B, case.L).astype(np.float64)
    n_b = np.maximum(m.sum(1), 1.0)
    s_b = (m * x).sum(1) / n_b
    ratio_b, pg_b, clip_b = oracle.ppo_clip_terms(s_b, case.adv.astype(np.float64), case.eps_low, case.eps_high)
    assert (kink_distance(s_b, case.eps_low, case.eps_high) > 1e-4).all()
    assert_rel(fwd["seq_ratio"].cpu().numpy(), ratio_b, "seq_ratio")
    assert_rel(fwd["loss"].cpu().numpy(), np.repeat(pg_b, case.L), "loss (all rows)")
    assert np.array_equal(fwd["is_clipped"].cpu().numpy().astype(bool), np.repeat(clip_b, case.L))
    o.update(is_clipped=np.repeat(clip_b, case.L), seq_ratio=ratio_b, seq_n=n_b)
    g = oracle.grpo_dlogp(o, None, case.adv, case.mask, case.dloss, case.B, case.L, 0.0, "sequence")
    zr_np = zr.cpu().numpy().astype(bool)
    assert np.array_equal(zr_np, g == 0.0)
    say(f"  zero rows {zr_np.sum()} of {case.N}; clipped sequences {int(clip_b.sum())}")
    # sampled rows against the full oracle (lse, entropy, dlogits)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, case.N - 1], rng.integers(0, case.N, 40),
                                     np.flatnonzero(~zr_np)[:8]]))
    z64 = oracle.decode_bf16(case.logits[rows])
    _, lse = oracle.log_softmax_stats(z64, case.temperature)
    assert_rel(fwd["lse"].cpu().numpy()[rows], lse, "lse (sampled)")
    assert_rel(fwd["entropy"].cpu().numpy()[rows], oracle.entropy_from_logits(z64), "entropy (sampled)")
    dz_o = oracle.dlogits_from_dlogp(z64, case.ids[rows], lse, g[rows], case.temperature)
    got = dev_to_f64(dz[torch.from_numpy(rows).cuda()])
    assert_bf16_dz(got, dz_o)
    # every row: zero rows +0.0, row sums ~ 0
    zb = dz[torch.from_numpy(zr_np).cuda()].view(torch.int16)
    assert int((zb != 0).sum()) == 0
    rs = dz.float().sum(dim=1).abs().cpu().numpy()
    assert (rs <= 1e-2 * np.abs(g) / case.temperature + 1e-6).all()
    _, dz2, _ = run_grpo_gpu(lib, t, inp, force_dense=True)
    assert torch.equal(dz, dz2)


# ---------------------------------------------------------------------------
# entropy_from_logits and selective_log_softmax: N=65536, V=32000, bf16
# ---------------------------------------------------------------------------
def test_entropy_and_selective_logsoftmax_full():
    lib = require_gpu()
    case = synth.row_case()
    say("entropy + selective log-softmax fwd/bwd: N=65536 V=32000 bf16 (contiguous and row stride 2V)")
    t = logits_to_dev(case.logits, "bf16")
    ids = dev(case.ids)
    grad = dev(case.grad)
    H = lib.entropy_from_logits(t)
    logp, lse = lib.selective_log_softmax(t, ids)
    dz = lib.selective_log_softmax_bwd(t, ids, lse, grad)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(case.N - 32, case.N),
                                     rng.integers(0, case.N, 192)]))
    z64 = oracle.decode_bf16(case.logits[rows])
    lp_o, lse_o = oracle.selective_log_softmax(z64, case.ids[rows])
    assert_rel(H.cpu().numpy()[rows], oracle.entropy_from_logits(z64), "entropy (sampled)")
    assert_rel(logp.cpu().numpy()[rows], lp_o, "logp (sampled)")
    assert_rel(lse.cpu().numpy()[rows], lse_o, "lse (sampled)")
    dz_o = oracle.selective_log_softmax_bwd(z64, case.ids[rows], case.grad[rows])
    assert_bf16_dz(dev_to_f64(dz[torch.from_numpy(rows).cuda()]), dz_o)
    # every row: bounds and row sums
    Hn = H.cpu().numpy()
    assert (Hn >= -1e-6).all() and (Hn <= math.log(case.V) * (1 + 1e-6)).all()
    assert (logp.cpu().numpy() <= 1e-6).all()
    rs = dz.float().sum(1).abs().cpu().numpy()
    assert (rs <= 1e-2 * np.abs(case.grad) + 1e-6).all()
    # strided input: rows of a [N, 2V] buffer whose other half is a NaN sentinel
    buf = torch.empty((case.N, 2 * case.V), dtype=torch.bfloat16, device="cuda")
    buf[:, case.V:] = float("nan")
    buf[:, :case.V] = t
    sview = buf[:, :case.V]
    sentinel = buf[:, case.V:].contiguous().view(torch.int16).clone()
    del t
    H2 = lib.entropy_from_logits(sview)
    logp2, lse2 = lib.selective_log_softmax(sview, ids)
    dz2 = lib.selective_log_softmax_bwd(sview, ids, lse2, grad)
    torch.cuda.synchronize()
    assert torch.equal(H2, H) and torch.equal(logp2, logp) and torch.equal(lse2, lse)
    assert torch.equal(dz2.view(torch.int16), dz.view(torch.int16))
    assert torch.equal(buf[:, case.V:].contiguous().view(torch.int16), sentinel)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,ld_extra", [(1, 0), (17, 0), (1003, 0), (4099, 0), (1003, 1), (640, 3),
                                        (1, 7), (1003, 5), (4099, 5), (16003, 5), (40003, 5)])
def test_ragged_and_strided_rows(dtype, V, ld_extra):
    """Tails shorter than one 128-bit vector, V = 1, and row strides that are
    not 16-byte multiples (element-wise path); ragged rows on 16-byte pitches
    (ld_extra 5 and 7, fp32 1003 + 1) take the vector path with a tail."""
    lib = require_gpu()
    say(f"edge: dtype {dtype} V={V} ld=V+{ld_extra}")
    B, L = 3, 5
    rng = np.random.default_rng(V + ld_extra)
    zf = (rng.standard_normal((B * L, V + ld_extra)) * 2.0).astype(np.float32)
    zb = synth.f32_to_bf16_bits(zf) if dtype == "bf16" else zf
    full = logits_to_dev(zb, dtype)
    t = full[:, :V]
    z64 = oracle.to_f64(zb, dtype)[:, :V]
    ids = rng.integers(0, V, B * L).astype(np.int64)
    adv = np.array([0.7, 0.0, -1.2], np.float32)
    lp, _ = oracle.selective_log_softmax(z64, ids, 0.9)
    case = synth.GrpoCase(name="edge", B=B, L=L, V=V, dtype=dtype, logits=None, ids=ids, adv=adv,
                          mask=np.ones(B * L, np.uint8), old_noise=rng.standard_normal(B * L) * 0.2,
                          ref_noise=rng.standard_normal(B * L) * 0.1,
                          dloss=np.ones(B * L, np.float32), temperature=0.9, beta=0.04,
                          eps_low=0.2, eps_high=0.28, level="token")
    inp = GrpoInputs(case, lp)
    fwd, dz, zr = run_grpo_gpu(lib, t, inp)
    o, g = oracle_expectations(inp, z64, fwd)
    check_forward(case, o, fwd, ref=inp.ref)
    check_backward(case, o, g, dz, zr, z64, inp)
    H = lib.entropy_from_logits(t, temperature=0.9)
    assert_rel(H.cpu().numpy(), oracle.entropy_from_logits(z64, 0.9), "entropy")


@pytest.mark.parametrize("level", ["token", "sequence"])
@pytest.mark.parametrize("dtype,V", [("bf16", 32779), ("bf16", 65536), ("f32", 16388),
                                     ("f32", 16391)])
def test_split_rows_backward(dtype, V, level):
    """Long rows: the backward takes one workgroup per chunk of a row (512
    vectors at token level, 4096 at sequence level).  4097 vectors (the last
    chunk one vector, with or without a tail of 3 elements) and 8192 (whole
    chunks only); the sampled ids sit on the row's first and last element
    and on both sides of the 4096-vector boundary (a chunk boundary at both
    levels); the
    second sequence has advantage 0 (beta 0: zero rows; the old log-probs
    close enough that no token of the first is clipped).  Checked against
    the oracle, the zero rows' flags and +0.0, the forced-dense result equal
    to the skipping one, the pad columns of a wider output untouched, and
    rows with an out-of-range id all NaN."""
    lib = require_gpu()
    say(f"split rows: dtype {dtype} V={V} level {level}")
    B, L = 2, 4
    es = 2 if dtype == "bf16" else 4
    VE = 16 // es
    pad = (-V) % VE or VE  # a 16-byte row pitch: the vector path
    rng = np.random.default_rng(V + (1 if level == "token" else 2))
    zf = (rng.standard_normal((B * L, V + pad)) * 2.0).astype(np.float32)
    zb = synth.f32_to_bf16_bits(zf) if dtype == "bf16" else zf
    t = logits_to_dev(zb, dtype)[:, :V]
    z64 = oracle.to_f64(zb, dtype)[:, :V]
    edge = 4096 * VE  # first element of the second chunk
    ids = rng.integers(0, V, B * L).astype(np.int64)
    ids[:4] = [0, V - 1, edge - 1, edge]
    adv = np.array([0.9, 0.0], np.float32)
    lp, _ = oracle.selective_log_softmax(z64, ids, 0.9)
    case = synth.GrpoCase(name="split", B=B, L=L, V=V, dtype=dtype, logits=None, ids=ids, adv=adv,
                          mask=np.ones(B * L, np.uint8), old_noise=rng.standard_normal(B * L) * 0.01,
                          ref_noise=None, dloss=np.full(B * L, 1.0 / (B * L), np.float32),
                          temperature=0.9, beta=0.0, eps_low=0.2, eps_high=0.28, level=level)
    inp = GrpoInputs(case, lp)
    fwd, dz, zr = run_grpo_gpu(lib, t, inp)
    o, g = oracle_expectations(inp, z64, fwd)
    assert (g[4:] == 0.0).all() and (g[:4] != 0.0).all()
    check_forward(case, o, fwd)
    check_backward(case, o, g, dz, zr, z64, inp)
    d = inp.to_dev()
    kw = dict(ref_logp=None, mask=d["mask"], seq_ratio=fwd.get("seq_ratio"), temperature=0.9,
              beta=0.0, eps_low=0.2, eps_high=0.28, level=level)
    dense, _ = lib.grpo_logits_bwd(t, d["ids"], d["old_logp"], d["adv"], B, L, fwd["logp"],
                                   fwd["lse"], d["dloss"], force_dense=True, **kw)
    wide = torch.full((B * L, V + pad), float("nan"), dtype=t.dtype, device="cuda")
    sentinel = wide[:, V:].clone()
    lib.grpo_logits_bwd(t, d["ids"], d["old_logp"], d["adv"], B, L, fwd["logp"], fwd["lse"],
                        d["dloss"], dlogits=wide[:, :V], **kw)
    bad = ids.copy()
    bad[[1, 2, 5]] = [-1, V, -1]
    bad_t = dev(bad)
    nan_dz, _ = lib.grpo_logits_bwd(t, bad_t, d["old_logp"], d["adv"], B, L, fwd["logp"],
                                    fwd["lse"], d["dloss"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(dense, dz)
    assert np.array_equal(bits(wide[:, :V]), bits(dz))
    assert torch.equal(wide[:, V:].view(torch.int16) if es == 2 else wide[:, V:].view(torch.int32),
                       sentinel.view(torch.int16) if es == 2 else sentinel.view(torch.int32))
    n = dev_to_f64(nan_dz)
    assert np.isnan(n[[1, 2, 5]]).all()
    keep = [0, 3, 4, 6, 7]
    assert np.array_equal(bits(nan_dz)[keep], bits(dz)[keep])


@pytest.mark.parametrize("dtype,V,ld_extra", [("f32", 17, 0), ("bf16", 1003, 0), ("bf16", 1003, 1),
                                             ("bf16", 32000, 0), ("f32", 4099, 5),
                                             ("bf16", 151936, 0)])
@pytest.mark.parametrize("T", [0.05, 0.1])
def test_low_temperature_rows(dtype, V, ld_extra, T):
    """T = 0.05 and 0.1 with every other row sampling its most likely token,
    so logp is close to 0 and the 1e-6 floor of the bar binds: the GRPO
    forward and backward (two passes), the entropy, and the selective
    log-softmax forward and backward.  A lane's sums must be referenced to
    its exact max: referenced to the rounded product fl(m log2e / T) they
    carry an offset of up to half an ulp of it (7.6e-6 at m/T ~ 100), which
    lse and logp inherit.  bf16 dlogits reach |o| >= 4 here, where the bar is
    one bf16 ulp of the oracle value."""
    lib = require_gpu()
    say(f"low temperature: dtype {dtype} V={V} ld=V+{ld_extra} T={T}")
    B, L = 2, 4
    rng = np.random.default_rng(V + 7 * ld_extra + int(100 * T))
    zf = (rng.standard_normal((B * L, V + ld_extra)) * 2.0).astype(np.float32)
    zb = synth.f32_to_bf16_bits(zf) if dtype == "bf16" else zf
    t = logits_to_dev(zb, dtype)[:, :V]
    z64 = oracle.to_f64(zb, dtype)[:, :V]
    ids = rng.integers(0, V, B * L).astype(np.int64)
    ids[::2] = z64[::2].argmax(axis=1)
    lp, _ = oracle.selective_log_softmax(z64, ids, T)
    case = synth.GrpoCase(name="low-T", B=B, L=L, V=V, dtype=dtype, logits=None, ids=ids,
                          adv=np.array([0.7, -1.2], np.float32), mask=np.ones(B * L, np.uint8),
                          old_noise=rng.standard_normal(B * L) * 0.2,
                          ref_noise=rng.standard_normal(B * L) * 0.1,
                          dloss=np.ones(B * L, np.float32), temperature=T, beta=0.04,
                          eps_low=0.2, eps_high=0.28, level="token")
    inp = GrpoInputs(case, lp)
    fwd, dz, zr = run_grpo_gpu(lib, t, inp)
    o, g = oracle_expectations(inp, z64, fwd)
    check_forward(case, o, fwd, ref=inp.ref)
    check_backward(case, o, g, dz, zr, z64, inp)
    H = lib.entropy_from_logits(t, temperature=T)
    lpg, lseg = lib.selective_log_softmax(t, dev(ids), temperature=T)
    gr = rng.standard_normal(B * L).astype(np.float32)
    dzs = lib.selective_log_softmax_bwd(t, dev(ids), lseg, dev(gr), temperature=T)
    torch.cuda.synchronize()
    lp_o, lse_o = oracle.selective_log_softmax(z64, ids, T)
    assert_rel(H.cpu().numpy(), oracle.entropy_from_logits(z64, T), "entropy")
    assert_rel(lpg.cpu().numpy(), lp_o, "selective logp")
    assert_rel(lseg.cpu().numpy(), lse_o, "selective lse")
    dzs_o = oracle.selective_log_softmax_bwd(z64, ids, gr, T)
    if dtype == "bf16":
        assert_bf16_dz(dev_to_f64(dzs), dzs_o, "selective dlogits")
    else:
        tol = np.abs(gr / T)[:, None] * (1e-5 * np.abs(lse_o) + 2e-6)[:, None]
        assert (np.abs(dev_to_f64(dzs) - dzs_o) <= tol).all(), "selective fp32 dlogits"


def test_empty_rows_are_noop():
    lib = require_gpu()
    say("edge: zero rows")
    t = torch.empty((0, 100), dtype=torch.bfloat16, device="cuda")
    assert lib.entropy_from_logits(t).numel() == 0
    lp, lse = lib.selective_log_softmax(t, torch.empty(0, dtype=torch.int64, device="cuda"))
    assert lp.numel() == 0


def test_invalid_ids_give_nan_and_count():
    lib = require_gpu()
    say("edge: out-of-range ids")
    case, z64, inp = _tiny("a")
    t = logits_to_dev(case.logits, "f32")
    d = inp.to_dev()
    bad = case.ids.copy()
    bad[3] = -1
    bad[7] = case.V
    d["ids"] = dev(bad)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fwd = lib.grpo_logits_fwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L,
                              ref_logp=d["ref_logp"], temperature=1.0, beta=case.beta,
                              err_count=err, gathered=True)
    dzt, _ = lib.grpo_logits_bwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L,
                                 fwd["logp"], fwd["lse"], d["dloss"], ref_logp=d["ref_logp"],
                                 temperature=1.0, beta=case.beta)
    torch.cuda.synchronize()
    assert int(err.item()) == 2
    lp = fwd["logp"].cpu().numpy()
    assert np.isnan(lp[[3, 7]]).all() and np.isfinite(np.delete(lp, [3, 7])).all()
    dzn = dzt.cpu().numpy()
    assert np.isnan(dzn[[3, 7]]).all() and np.isfinite(np.delete(dzn, [3, 7], axis=0)).all()


def test_in_place_backward():
    lib = require_gpu()
    say("edge: in-place dlogits")
    case, inp = _token_case(False, "sum")
    t = logits_to_dev(case.logits, "bf16")
    fwd, dz, zr = run_grpo_gpu(lib, t, inp)
    d = inp.to_dev()
    lib.grpo_logits_bwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L, fwd["logp"],
                        fwd["lse"], d["dloss"], mask=d["mask"], temperature=case.temperature,
                        beta=case.beta, eps_low=case.eps_low, eps_high=case.eps_high, dlogits=t)
    torch.cuda.synchronize()
    assert torch.equal(t.view(torch.int16), dz.view(torch.int16))


def test_nan_logits_propagate():
    lib = require_gpu()
    say("edge: NaN in a row")
    rng = np.random.default_rng(3)
    z = rng.standard_normal((4, 300)).astype(np.float32)
    z[1, 17] = np.nan
    t = logits_to_dev(z, "f32")
    H = lib.entropy_from_logits(t).cpu().numpy()
    lp, lse = lib.selective_log_softmax(t, dev(np.array([0, 1, 2, 3], np.int64)))
    assert np.isnan(H[1]) and np.isnan(lse.cpu().numpy()[1])
    assert np.isfinite(np.delete(H, 1)).all()


@pytest.mark.parametrize("with_ref", [False, True])
def test_sequence_level_partial_masks(with_ref):
    """Sequence level with completion masks of lengths 12, 0, 1 and 7 (an
    empty sequence, a one-token sequence): the mask-weighted mean log-ratio,
    its clip and the spread gradient against the oracle; every row."""
    lib = require_gpu()
    say(f"sequence level with partial masks (lengths 12, 0, 1, 7), ref={'noise' if with_ref else 'none'}")
    B, L, V = 4, 12, 300
    rng = np.random.default_rng(61)
    z = (rng.standard_normal((B * L, V)) * 2.0).astype(np.float32)
    z64 = z.astype(np.float64)
    ids = rng.integers(0, V, B * L).astype(np.int64)
    T = 0.8
    lp, _ = oracle.selective_log_softmax(z64, ids, T)
    lengths = np.array([12, 0, 1, 7])
    mask = (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8).reshape(-1)
    case = synth.GrpoCase(name="seq-masks", B=B, L=L, V=V, dtype="f32", logits=z, ids=ids,
                          adv=np.array([0.9, -0.4, 1.3, -1.0], np.float32), mask=mask,
                          old_noise=np.repeat(rng.standard_normal(B) * 0.4, L),
                          ref_noise=rng.standard_normal(B * L) * 0.1 if with_ref else None,
                          dloss=mask.astype(np.float32), temperature=T, beta=0.04,
                          eps_low=0.2, eps_high=0.28, level="sequence")
    inp = GrpoInputs(case, lp)
    fwd, dz, zr = run_grpo_gpu(lib, logits_to_dev(z, "f32"), inp)
    o, g = oracle_expectations(inp, z64, fwd)
    check_forward(case, o, fwd, ref=inp.ref)
    check_backward(case, o, g, dz, zr, z64, inp)
    # the empty sequence (and the masked tail of the others) carries no
    # policy gradient; without a reference model its rows are exactly zero
    if not with_ref:
        assert zr.cpu().numpy()[mask == 0].all()
