"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each pin is chosen so that a plausible slip in the oracle fails at least one:
  * library routines: log-sum-exp (scipy.special.logsumexp), entropy
    (scipy.stats.entropy of scipy.special.softmax);
  * hand-derived closed forms in tests/golden/closed_forms.json;
  * invariants: 0 <= H <= log V, rows of dlogits sum to 0, exact +0 rows,
    k3 >= 0 and k3 ~ d^2/2, shift and temperature identities;
  * central finite differences of sum(dloss * loss) in the logits (token and
    sequence level, T != 1, beta on/off, no reference) and, for the fused
    linear variant, in the hidden states and in the LM-head weight.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import synth
from case_weights import fill_dloss

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _gold():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# input decoding
# ---------------------------------------------------------------------------
def test_decode_bf16_every_pattern_matches_torch():
    """All 65536 bf16 bit patterns decode to the value torch's bfloat16 ->
    float32 conversion gives (NaN patterns to NaN)."""
    import torch
    pat = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(pat)
    ref = torch.from_numpy(pat.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # sign of zero kept
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0x0000])


def test_decode_bf16_hand_values():
    """Patterns whose values follow from the binary32 layout by hand."""
    pats = np.array([0x3F80, 0xBF80, 0x4049, 0x4000, 0x3F00, 0x0001, 0x0080, 0x7F80, 0xFF80,
                     0x7F7F, 0x3F81], np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0, 0.5, 2.0 ** -133, 2.0 ** -126, np.inf, -np.inf,
            (2 - 2 ** -7) * 2.0 ** 127, 1 + 2 ** -7]
    assert oracle.decode_bf16(pats).tolist() == want



def test_to_f64_per_dtype():
    """fp32 logits widen exactly (every float32 is a float64); bf16 logits
    arrive as their bit patterns and come back as the values those patterns
    stand for, checked here by hand, not through decode_bf16."""
    f32 = np.array([[1.0, -2.5, 3.0e38, 1.0e-45], [0.1, -0.0, 7.0, 2.0 ** -20]], np.float32)
    got = oracle.to_f64(f32, "f32")
    assert got.dtype == np.float64 and got.shape == f32.shape
    assert np.array_equal(got, f32.astype(np.float64)) and np.signbit(got[1, 1])
    bits = np.array([[0x3F80, 0xC020], [0x4120, 0x0000]], np.uint16)   # 1, -2.5, 10, +0
    assert oracle.to_f64(bits, "bf16").tolist() == [[1.0, -2.5], [10.0, 0.0]]


# ---------------------------------------------------------------------------
# library routines
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1.0, 0.7, 1.9])
def test_lse_matches_scipy(T):
    rng = np.random.default_rng(1)
    z = rng.standard_normal((7, 513)) * 3.0
    _, lse = oracle.log_softmax_stats(z, T)
    ref = scipy.special.logsumexp(z / T, axis=1)
    np.testing.assert_allclose(lse, ref, rtol=1e-14, atol=1e-14)
    ref2 = np.logaddexp.reduce(z / T, axis=1)
    np.testing.assert_allclose(lse, ref2, rtol=1e-13)


@pytest.mark.parametrize("T", [1.0, 0.9])
def test_entropy_matches_scipy(T):
    rng = np.random.default_rng(2)
    z = rng.standard_normal((300, 257)) * 2.0
    H = oracle.entropy_from_logits(z, T)
    p = scipy.special.softmax(z / T, axis=1)
    np.testing.assert_allclose(H, scipy.stats.entropy(p, axis=1), rtol=1e-12)


def test_selective_logsoftmax_matches_scipy():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((9, 100)) * 4.0
    idx = rng.integers(0, 100, 9)
    logp, lse = oracle.selective_log_softmax(z, idx, 1.3)
    ref = scipy.special.log_softmax(z / 1.3, axis=1)[np.arange(9), idx]
    np.testing.assert_allclose(logp, ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# closed forms (hand-derived fixture)
# ---------------------------------------------------------------------------
def _four_class(T):
    return (T * np.log(np.array([1.0, 2.0, 3.0, 4.0])))[None, :]


def test_golden_four_class_row():
    g = _gold()["four_class_row"]
    T = g["temperature"]
    z = _four_class(T)
    logp, lse = oracle.selective_log_softmax(z, np.array([g["index"]]), T)
    assert abs(lse[0] - g["lse_value"]) < 1e-14
    assert abs(logp[0] - g["logp_value"]) < 1e-14
    H = oracle.entropy_from_logits(z, T)
    assert abs(H[0] - g["entropy_value"]) < 1e-14
    dz = oracle.selective_log_softmax_bwd(z, np.array([g["index"]]), np.array([g["grad_logp"]]), T)
    np.testing.assert_allclose(dz[0], g["dlogits_value"], atol=1e-15)


@pytest.mark.parametrize("case", _gold()["token_cases"]["cases"], ids=lambda c: c["name"])
def test_golden_token_cases(case):
    T = 2.0
    z = _four_class(T)
    ids = np.array([2])
    logp = math.log(0.3)
    old = np.array([logp - math.log(case["ratio"])])
    ref = None if case["ref_minus_logp"] is None else np.array([logp + math.log(2.0)])
    args = dict(z=z, ids=ids, old_logp=old, ref_logp=ref, adv=np.array([case["adv"]]),
                mask=None, B=1, L=1, temperature=T, beta=case["beta"],
                eps_low=case["eps_low"], eps_high=case["eps_high"], level="token")
    fwd = oracle.grpo_forward(**args)
    assert abs(fwd["loss"][0] - case["loss_value"]) < 1e-13
    assert abs(fwd["kl"][0] - case["kl_value"]) < 1e-13
    assert bool(fwd["is_clipped"][0]) == case["is_clipped"]
    dz, g, zero = oracle.grpo_backward(dloss=np.array([1.0]), **args)
    assert abs(g[0] - case["dlogp_value"]) < 1e-13
    np.testing.assert_allclose(dz[0], case["dlogits_value"], atol=1e-14)
    assert bool(zero[0]) == (case["dlogp_value"] == 0.0)


@pytest.mark.parametrize("case", _gold()["sequence_cases"]["cases"], ids=lambda c: c["name"])
def test_golden_sequence_cases(case):
    T = 2.0
    z = np.repeat(_four_class(T), 2, axis=0)
    ids = np.array([2, 2])
    logp = math.log(0.3)
    old = np.array([logp - math.log(r) for r in case["token_ratios"]])
    args = dict(z=z, ids=ids, old_logp=old, ref_logp=None, adv=np.array([2.0]),
                mask=np.array(case["mask"], np.uint8), B=1, L=2, temperature=T, beta=0.0,
                eps_low=0.2, eps_high=0.2, level="sequence")
    fwd = oracle.grpo_forward(**args)
    assert abs(fwd["seq_ratio"][0] - case["seq_ratio_value"]) < 1e-14
    np.testing.assert_allclose(fwd["loss"], case["loss_value"], atol=1e-13)
    assert not fwd["is_clipped"].any() if not case["is_clipped"] else fwd["is_clipped"].all()
    dz, g, zero = oracle.grpo_backward(dloss=np.array(case["dloss"]), **args)
    np.testing.assert_allclose(g, case["dlogp_value"], atol=1e-13)
    assert (dz[np.array(case["dlogp_value"]) == 0.0] == 0.0).all()


# ---------------------------------------------------------------------------
# closed forms and invariants on random rows
# ---------------------------------------------------------------------------
def test_uniform_row():
    V = 1000
    z = np.full((3, V), 1.7)
    logp, _ = oracle.selective_log_softmax(z, np.array([0, 5, 999]), 0.8)
    np.testing.assert_allclose(logp, -math.log(V), rtol=1e-14)
    np.testing.assert_allclose(oracle.entropy_from_logits(z, 0.8), math.log(V), rtol=1e-14)


def test_temperature_and_shift_identities():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((5, 300)) * 2.0
    idx = rng.integers(0, 300, 5)
    a, _ = oracle.selective_log_softmax(z, idx, 0.6)
    b, _ = oracle.selective_log_softmax(z / 0.6, idx, 1.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    c, _ = oracle.selective_log_softmax(z + rng.standard_normal((5, 1)) * 10.0, idx, 0.6)
    np.testing.assert_allclose(a, c, rtol=1e-12)
    np.testing.assert_allclose(oracle.entropy_from_logits(z, 0.6),
                               oracle.entropy_from_logits(z + 3.0, 0.6), rtol=1e-12)


def test_entropy_bounds():
    rng = np.random.default_rng(5)
    for scale in (0.01, 1.0, 10.0, 100.0):
        z = rng.standard_normal((50, 777)) * scale
        H = oracle.entropy_from_logits(z)
        assert (H >= -1e-12).all() and (H <= math.log(777) + 1e-12).all()


def test_k3_properties():
    d = np.linspace(-3, 3, 601)
    assert (oracle.k3(d) >= 0).all()
    small = np.array([1e-3, -2e-4, 5e-6])
    np.testing.assert_allclose(oracle.k3(small), small ** 2 / 2, rtol=2e-3)


def _tiny_inputs(variant):
    case = fill_dloss(synth.tiny_case(variant))
    z = case.logits.astype(np.float64)
    logp_true, _ = oracle.selective_log_softmax(z, case.ids, case.temperature)
    old = synth.add_noise_f32(logp_true, case.old_noise).astype(np.float64)
    ref = None if case.ref_noise is None else synth.add_noise_f32(logp_true, case.ref_noise).astype(np.float64)
    return case, z, old, ref


def _args(case, z, old, ref):
    return dict(z=z, ids=case.ids, old_logp=old, ref_logp=ref, adv=case.adv, mask=case.mask,
                B=case.B, L=case.L, temperature=case.temperature, beta=case.beta,
                eps_low=case.eps_low, eps_high=case.eps_high, level=case.level)


def test_ratio_one_and_ref_equal_policy():
    case, z, _, _ = _tiny_inputs("a")
    logp, _ = oracle.selective_log_softmax(z, case.ids, case.temperature)
    a = _args(case, z, logp.copy(), logp.copy())
    fwd = oracle.grpo_forward(**a)
    A_row = np.repeat(case.adv.astype(np.float64), case.L)
    np.testing.assert_allclose(fwd["loss"], -A_row, atol=1e-12)   # ratio 1, k3 = 0
    assert np.abs(fwd["kl"]).max() < 1e-12
    dz, g, _ = oracle.grpo_backward(dloss=case.dloss, **a)
    np.testing.assert_allclose(g, A_row * -1.0 * case.dloss, atol=1e-12)


@pytest.mark.parametrize("variant", ["a", "b", "c", "s", "t"])
def test_dlogits_rows_sum_to_zero_and_zero_rows(variant):
    case, z, old, ref = _tiny_inputs(variant)
    dz, g, zero = oracle.grpo_backward(dloss=case.dloss, **_args(case, z, old, ref))
    scale = np.abs(g) / case.temperature
    assert (np.abs(dz.sum(axis=1)) <= 1e-14 * np.maximum(scale, 1e-300) * 10).all()
    # rows with dlogp == 0 are +0.0 (sign bit clear)
    assert not np.signbit(dz[zero]).any() and (dz[zero] == 0.0).all()


def test_tiny_zero_advantage_rows():
    """Sequence 1 has advantage 0.  With beta = 0 or no reference its rows are
    exactly zero; with beta > 0 and a reference they carry only the KL
    gradient beta * (1 - e^{ref - logp}) * dloss / T * (onehot - p)."""
    for variant in ("b", "c"):
        case, z, old, ref = _tiny_inputs(variant)
        dz, g, zero = oracle.grpo_backward(dloss=case.dloss, **_args(case, z, old, ref))
        assert zero[case.L:].all() and (dz[case.L:] == 0.0).all()
    case, z, old, ref = _tiny_inputs("a")
    a = _args(case, z, old, ref)
    fwd = oracle.grpo_forward(**a)
    dz, g, zero = oracle.grpo_backward(dloss=case.dloss, **a)
    r = slice(case.L, 2 * case.L)
    expect_g = case.beta * (1.0 - np.exp(ref[r] - fwd["logp"][r])) * case.dloss[r]
    np.testing.assert_allclose(g[r], expect_g, rtol=1e-13)
    assert not zero[r].any()


def test_reinforce_special_case():
    """beta = 0 and no token clipped: dz = -ratio*A*dloss/T*(onehot - p) (REINFORCE with an importance ratio)."""
    case, z, old, _ = _tiny_inputs("b")
    a = _args(case, z, old, None)
    a["eps_low"] = a["eps_high"] = 1e9
    fwd = oracle.grpo_forward(**a)
    assert not fwd["is_clipped"].any()
    dz, _, _ = oracle.grpo_backward(dloss=case.dloss, **a)
    p = scipy.special.softmax(z / case.temperature, axis=1)
    onehot = np.eye(case.V)[case.ids]
    coef = -np.exp(fwd["logp"] - old) * np.repeat(case.adv, case.L) * case.dloss / case.temperature
    expect = coef[:, None] * (onehot - p)
    expect[coef == 0.0] = 0.0
    np.testing.assert_allclose(dz, expect, atol=1e-15)


# ---------------------------------------------------------------------------
# finite differences
# ---------------------------------------------------------------------------
def _kink_distance(case, fwd, old):
    lo, hi = math.log(1 - case.eps_low), math.log(1 + case.eps_high)
    if case.level == "token":
        x = fwd["logp"] - old
    else:
        x = fwd["seq_logratio"]
    return np.minimum(np.abs(x - lo), np.abs(x - hi)).min()


def _loss_sum(case, z, old, ref):
    fwd = oracle.grpo_forward(**_args(case, z, old, ref))
    return float((case.dloss.astype(np.float64) * fwd["loss"]).sum())


@pytest.mark.parametrize("variant", ["a", "b", "c", "s", "t"])
def test_grpo_gradient_finite_differences(variant):
    case, z, old, ref = _tiny_inputs(variant)
    if variant == "s":
        # a sequence-level case with the KL term on as well
        case.beta = 0.04
        ref = synth.add_noise_f32(oracle.selective_log_softmax(z, case.ids)[0],
                                  case.ref_noise if case.ref_noise is not None else
                                  np.zeros(case.N)).astype(np.float64)
    a = _args(case, z, old, ref)
    fwd = oracle.grpo_forward(**a)
    assert _kink_distance(case, fwd, old) > 1e-4
    dz, _, _ = oracle.grpo_backward(dloss=case.dloss, **a)
    rng = np.random.default_rng(11)
    checked = 0
    for r in range(case.N):
        cols = {int(case.ids[r]), int(np.argmax(z[r]))} | set(rng.integers(0, case.V, 4).tolist())
        for j in cols:
            h = 1e-5 * max(1.0, abs(z[r, j]))
            zp = z.copy(); zp[r, j] += h
            zm = z.copy(); zm[r, j] -= h
            fd = (_loss_sum(case, zp, old, ref) - _loss_sum(case, zm, old, ref)) / (2 * h)
            tol = 1e-6 * max(np.abs(dz[r]).max(), 1e-3) + 1e-9
            assert abs(fd - dz[r, j]) <= tol, (variant, r, j, fd, dz[r, j])
            checked += 1
    assert checked > 100


def test_selective_logsoftmax_bwd_finite_differences():
    rng = np.random.default_rng(6)
    z = rng.standard_normal((4, 50)) * 2.0
    idx = rng.integers(0, 50, 4)
    gam = rng.standard_normal(4)
    T = 0.8
    dz = oracle.selective_log_softmax_bwd(z, idx, gam, T)
    f = lambda zz: float((gam * oracle.selective_log_softmax(zz, idx, T)[0]).sum())
    for r in range(4):
        for j in range(50):
            h = 1e-5
            zp = z.copy(); zp[r, j] += h
            zm = z.copy(); zm[r, j] -= h
            assert abs((f(zp) - f(zm)) / (2 * h) - dz[r, j]) < 1e-9


def _fused_tiny():
    B, L, H, V = 2, 4, 16, 64
    case = fill_dloss(synth.fused_case(B=B, L=L, H=H, V=V, dloss="sum"))
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight) * 25.0   # logits O(1) so the ratios move
    T = case.temperature
    logp, _ = oracle.selective_log_softmax(h @ W.T, case.ids, T)
    old = synth.add_noise_f32(logp, case.old_noise).astype(np.float64)
    ref = synth.add_noise_f32(logp, case.ref_noise).astype(np.float64)
    return case, h, W, old, ref


def test_fused_linear_finite_differences():
    case, h, W, old, ref = _fused_tiny()
    args = (case.ids, old, ref, case.adv, case.mask, case.dloss, case.B, case.L,
            case.temperature, case.beta, case.eps_low, case.eps_high)
    loss, gh, gW = oracle.fused_linear_grpo(h, W, *args, chunk_seqs=1)
    f = lambda hh, WW: oracle.fused_linear_loss(hh, WW, *args)
    assert abs(loss - f(h, W)) < 1e-12
    rng = np.random.default_rng(7)
    for _ in range(40):
        r, k = rng.integers(0, h.shape[0]), rng.integers(0, h.shape[1])
        eps = 1e-6
        hp = h.copy(); hp[r, k] += eps
        hm = h.copy(); hm[r, k] -= eps
        fd = (f(hp, W) - f(hm, W)) / (2 * eps)
        assert abs(fd - gh[r, k]) <= 1e-6 * max(np.abs(gh).max(), 1e-3), (r, k, fd, gh[r, k])
        v, k = rng.integers(0, W.shape[0]), rng.integers(0, W.shape[1])
        Wp = W.copy(); Wp[v, k] += eps
        Wm = W.copy(); Wm[v, k] -= eps
        fd = (f(h, Wp) - f(h, Wm)) / (2 * eps)
        assert abs(fd - gW[v, k]) <= 1e-6 * max(np.abs(gW).max(), 1e-3), (v, k, fd, gW[v, k])


def test_fused_linear_chunk_invariance_and_composition():
    case, h, W, old, ref = _fused_tiny()
    args = (case.ids, old, ref, case.adv, case.mask, case.dloss, case.B, case.L,
            case.temperature, case.beta, case.eps_low, case.eps_high)
    l1, gh1, gW1 = oracle.fused_linear_grpo(h, W, *args, chunk_seqs=1)
    l2, gh2, gW2 = oracle.fused_linear_grpo(h, W, *args, chunk_seqs=2)
    assert abs(l1 - l2) < 1e-12
    np.testing.assert_allclose(gh1, gh2, atol=1e-14)
    np.testing.assert_allclose(gW1, gW2, atol=1e-14)
    # unfused composition: logits -> GRPO backward -> two products
    z = h @ W.T
    dz, _, _ = oracle.grpo_backward(z, case.ids, old, ref, case.adv, case.mask, case.dloss,
                                    case.B, case.L, case.temperature, case.beta, case.eps_low,
                                    case.eps_high)
    np.testing.assert_allclose(gh1, dz @ W, atol=1e-14)
    np.testing.assert_allclose(gW1, dz.T @ h, atol=1e-14)


def test_ppo_clip_truth_table():
    """The clipped surrogate's four quadrants, a ratio inside the interval and
    a zero advantage, with eps_low 0.2 and eps_high 0.28 (interval [0.8,
    1.28]); expected loss and clip flag worked out by hand from
    pg = -min(r A, clip(r) A):
      r 1.5, A  2: min(3.0, 2.56)   -> pg -2.56, clipped
      r 0.5, A  2: min(1.0, 1.6)    -> pg -1.0,  not clipped
      r 0.5, A -2: min(-1.0, -1.6)  -> pg  1.6,  clipped
      r 1.5, A -2: min(-3.0, -2.56) -> pg  3.0,  not clipped
      r 1.1, A  2: both 2.2         -> pg -2.2,  not clipped (a tie keeps the gradient)
      r 1.5, A  0: both 0           -> pg  0,    not clipped"""
    r = np.array([1.5, 0.5, 0.5, 1.5, 1.1, 1.5])
    A = np.array([2.0, 2.0, -2.0, -2.0, 2.0, 0.0])
    ratio, pg, clipped = oracle.ppo_clip_terms(np.log(r), A, 0.2, 0.28)
    assert np.allclose(ratio, r, rtol=1e-15, atol=0)
    assert np.allclose(pg, [-2.56, -1.0, 1.6, 3.0, -2.2, 0.0], rtol=1e-14, atol=1e-15)
    assert clipped.tolist() == [True, False, True, False, False, False]
