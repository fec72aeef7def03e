"""GPU parity of the steps either side of the row pass, through the C ABI:
the entropy backward, group-relative advantages and loss-reduction weights,
and a chain rewards -> advantages -> weights -> GRPO logits pass.

Bars: the entropy backward in fp32 within the error its inputs and fp32
arithmetic allow (|d| <= 1e-5 |o| + 2e-6 |g/T| p (1 + |log p| + |H|)), in
bf16 additionally within the output rounding (2^-8 |o|), rows with a zero
upstream gradient bit-exact +0.0; advantages within 1e-6 relative (fp64
sums, one fp32 rounding), exact zeros bit-exact; weights bit-exact against
the float32 rounding of the oracle's float64 reciprocals."""
import numpy as np
import pytest
import torch

import oracle
import synth
from case_weights import fill_dloss
from gpu_common import bits, dev, dev_to_f64, logits_to_dev, require_gpu, say

pytestmark = pytest.mark.gpu


def _entropy_inputs(z64, T):
    """Oracle lse and H (float64 -> float32) for the backward's inputs."""
    u, lse = oracle.log_softmax_stats(z64, T)
    H = oracle.entropy_from_logits(z64, T)
    return lse, H


def _entropy_bound(z64, T, g, lse, H):
    logp = z64 / T - lse[:, None]
    p = np.exp(logp)
    return 2e-6 * (np.abs(g) / T)[:, None] * p * (1.0 + np.abs(logp) + np.abs(H)[:, None])


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_entropy_bwd_fp32(T):
    lib = require_gpu()
    c = fill_dloss(synth.tiny_case("a"))
    say(f"entropy backward fp32: rows {c.N} V {c.V} T {T}")
    z64 = c.logits.astype(np.float64)
    rng = np.random.default_rng(21)
    g = rng.standard_normal(c.N).astype(np.float32)
    g[::5] = 0.0
    lse, H = _entropy_inputs(z64, T)
    lse32, H32 = lse.astype(np.float32), H.astype(np.float32)
    dz = lib.entropy_from_logits_bwd(dev(c.logits), dev(lse32), dev(H32), dev(g), temperature=T)
    torch.cuda.synchronize()
    want = oracle.entropy_from_logits_bwd(z64, g.astype(np.float64), T)
    got = dev_to_f64(dz)
    tol = 1e-5 * np.abs(want) + _entropy_bound(z64, T, g, lse, H)
    assert (np.abs(got - want) <= tol).all(), np.abs(got - want).max()
    zero = g == 0.0
    assert (bits(dz)[zero] == 0).all()


def test_entropy_bwd_bf16_strided_and_in_place():
    lib = require_gpu()
    rc = synth.row_case(N=96, V=3000)
    say("entropy backward bf16: 96 x 3000, strided [N, 2V] source, then in place")
    T = 0.9
    z64 = oracle.decode_bf16(rc.logits)
    g = rc.grad.copy()
    g[7] = 0.0
    lse, H = _entropy_inputs(z64, T)
    want = oracle.entropy_from_logits_bwd(z64, g.astype(np.float64), T)
    tol = 2.0 ** -8 * np.abs(want) + 1e-5 * np.abs(want) + _entropy_bound(z64, T, g, lse, H) + 1e-30
    wide = torch.zeros((rc.N, 2 * rc.V), dtype=torch.bfloat16, device="cuda")
    wide[:, :rc.V] = logits_to_dev(rc.logits, "bf16")
    view = wide[:, :rc.V]
    args = (dev(lse.astype(np.float32)), dev(H.astype(np.float32)), dev(g))
    dz = lib.entropy_from_logits_bwd(view, *args, temperature=T)
    torch.cuda.synchronize()
    got = dev_to_f64(dz)
    assert (np.abs(got - want) <= tol).all(), np.abs(got - want).max()
    assert (bits(dz)[7] == 0).all()
    # in place over the strided view (ld_out = ld = 2V)
    lib.entropy_from_logits_bwd(view, *args, temperature=T, dlogits=view)
    torch.cuda.synchronize()
    assert np.array_equal(bits(view), bits(dz))


@pytest.mark.parametrize("dtype,V", [("bf16", 32779), ("f32", 16391)])
def test_entropy_bwd_split_rows(dtype, V):
    """Rows of 4097 vectors with a 3-element tail on a 16-byte pitch: the
    entropy backward takes one workgroup per 4096-vector chunk of a row."""
    lib = require_gpu()
    say(f"entropy backward {dtype}: 10 x {V} (rows split into chunks)")
    N, T = 10, 0.8
    es = 2 if dtype == "bf16" else 4
    pad = (-V) % (16 // es)
    rng = np.random.default_rng(V)
    zf = (rng.standard_normal((N, V + pad)) * 2.0).astype(np.float32)
    zb = synth.f32_to_bf16_bits(zf) if dtype == "bf16" else zf
    t = logits_to_dev(zb, dtype)[:, :V]
    z64 = oracle.to_f64(zb, dtype)[:, :V]
    g = rng.standard_normal(N).astype(np.float32)
    g[3] = 0.0
    lse, H = _entropy_inputs(z64, T)
    dz = lib.entropy_from_logits_bwd(t, dev(lse.astype(np.float32)), dev(H.astype(np.float32)),
                                     dev(g), temperature=T)
    torch.cuda.synchronize()
    want = oracle.entropy_from_logits_bwd(z64, g.astype(np.float64), T)
    tol = 1e-5 * np.abs(want) + _entropy_bound(z64, T, g, lse, H) + 1e-30
    if dtype == "bf16":
        tol = tol + 2.0 ** -8 * np.abs(want)
    assert (np.abs(dev_to_f64(dz) - want) <= tol).all()
    assert (bits(dz)[3] == 0).all()


def test_entropy_bwd_ragged_unaligned_rows():
    """V = 1003 bf16: rows not 16-byte aligned take the element-wise path."""
    lib = require_gpu()
    rc = synth.row_case(N=24, V=1003)
    say("entropy backward bf16: 24 x 1003 (element-wise path)")
    T = 1.0
    z64 = oracle.decode_bf16(rc.logits)
    g = rc.grad.copy()
    lse, H = _entropy_inputs(z64, T)
    dz = lib.entropy_from_logits_bwd(logits_to_dev(rc.logits, "bf16"), dev(lse.astype(np.float32)),
                                     dev(H.astype(np.float32)), dev(g), temperature=T)
    torch.cuda.synchronize()
    want = oracle.entropy_from_logits_bwd(z64, g.astype(np.float64), T)
    tol = 2.0 ** -8 * np.abs(want) + 1e-5 * np.abs(want) + _entropy_bound(z64, T, g, lse, H) + 1e-30
    assert (np.abs(dev_to_f64(dz) - want) <= tol).all()


def test_entropy_bwd_after_gpu_forwards():
    """lse from selective_log_softmax and H from entropy_from_logits (the
    library's own forwards), then the backward: matches the oracle within
    the forwards' 1e-5 relative error propagated."""
    lib = require_gpu()
    rc = synth.row_case(N=64, V=32000)
    say("entropy backward on the library's own forward outputs: 64 x 32000 bf16")
    T = 1.0
    z = logits_to_dev(rc.logits, "bf16")
    ids = dev(rc.ids)
    _, lse = lib.selective_log_softmax(z, ids, temperature=T)
    H = lib.entropy_from_logits(z, temperature=T)
    g = dev(rc.grad)
    dz = lib.entropy_from_logits_bwd(z, lse, H, g, temperature=T)
    torch.cuda.synchronize()
    z64 = oracle.decode_bf16(rc.logits)
    want = oracle.entropy_from_logits_bwd(z64, rc.grad.astype(np.float64), T)
    lse_o, H_o = _entropy_inputs(z64, T)
    logp = z64 / T - lse_o[:, None]
    p = np.exp(logp)
    # d lse and d H of 1e-5 relative move dz by |g| p (|d lse| |log p + H - 1| + |d H|)
    prop = (np.abs(rc.grad) / T)[:, None] * p * (
        1e-5 * np.abs(lse_o)[:, None] * (np.abs(logp + H_o[:, None]) + 1) + 1e-5 * np.abs(H_o)[:, None])
    tol = 2.0 ** -8 * np.abs(want) + prop + _entropy_bound(z64, T, rc.grad, lse_o, H_o) + 1e-30
    assert (np.abs(dev_to_f64(dz) - want) <= tol).all()


@pytest.mark.parametrize("G", [1, 2, 4, 16, 64])
def test_group_advantages(G):
    lib = require_gpu()
    say(f"group advantages, groups of {G}")
    rng = np.random.default_rng(31 + G)
    n = 64 * G
    r = rng.standard_normal(n).astype(np.float32)
    r[:G] = 0.5                                    # all equal: exactly 0
    if G >= 2:
        r[G:2 * G] = rng.integers(0, 2, G)         # binary rewards
    for scale in (True, False):
        a = lib.grpo_group_advantages(dev(r), G, eps=1e-4, scale=scale)
        torch.cuda.synchronize()
        got = a.cpu().numpy().astype(np.float64)
        want = oracle.group_advantages(r.astype(np.float64), G, 1e-4, scale)
        zero = want == 0.0
        assert (bits(a)[zero] == 0).all()
        assert (np.abs(got - want) <= 1e-6 * np.abs(want)).all(), np.abs(got - want).max()


def test_group_advantages_nan_group():
    lib = require_gpu()
    say("group advantages: a NaN reward poisons its group only")
    r = np.array([1, 2, 3, 4, 5, np.nan, 7, 8], dtype=np.float32)
    a = lib.grpo_group_advantages(dev(r), 4).cpu().numpy()
    want = oracle.group_advantages(r.astype(np.float64), 4)
    assert np.isnan(a[4:]).all() and np.isnan(want[4:]).all()
    assert np.allclose(a[:4], want[:4], rtol=1e-6, atol=0)


@pytest.mark.parametrize("reduction", ["token", "sequence", "constant"])
@pytest.mark.parametrize("with_mask", [True, False])
def test_loss_weights(reduction, with_mask):
    lib = require_gpu()
    B, L = 37, 523
    say(f"loss weights: {reduction}, mask {'given' if with_mask else 'NULL'}, B {B} L {L}")
    rng = np.random.default_rng(41)
    lengths = rng.integers(0, L + 1, size=B)
    lengths[3] = 0
    mask = (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8).reshape(-1)
    w = lib.grpo_loss_weights(dev(mask) if with_mask else None, B, L, reduction)
    torch.cuda.synchronize()
    want = oracle.loss_weights(mask if with_mask else None, B, L, reduction).astype(np.float32)
    assert np.array_equal(bits(w), want.view(np.uint32))


def test_rewards_to_logits_chain():
    """Binary rewards in groups of 4 -> advantages -> token-mean weights ->
    grpo_logits_fwd_bwd, with no reference model: the sequences of a group
    whose rewards are all equal get advantage 0 and their rows take the zero
    path, bit-identical to the oracle's zero-row mask."""
    lib = require_gpu()
    c = fill_dloss(synth.grpo_token_case(B=8, L=64, V=2048))
    say("chain: rewards -> advantages -> weights -> single-pass GRPO, B=8 L=64 V=2048")
    rewards = np.array([1, 1, 1, 1, 0, 1, 0, 0], dtype=np.float32)
    adv = lib.grpo_group_advantages(dev(rewards), 4)
    w = lib.grpo_loss_weights(dev(c.mask), c.B, c.L, "token")
    z64 = oracle.decode_bf16(c.logits)
    logp_true, _ = oracle.selective_log_softmax(z64, c.ids, c.temperature)
    old = synth.add_noise_f32(logp_true, c.old_noise)
    kw = dict(temperature=c.temperature, beta=c.beta, eps_low=c.eps_low, eps_high=c.eps_high)
    out, dz, zr = lib.grpo_logits_fwd_bwd(logits_to_dev(c.logits, "bf16"), dev(c.ids), dev(old),
                                          adv, c.B, c.L, w, mask=dev(c.mask), **kw)
    torch.cuda.synchronize()
    adv_o = oracle.group_advantages(rewards.astype(np.float64), 4)
    assert (adv.cpu().numpy()[:4] == 0.0).all() and (adv_o[:4] == 0.0).all()
    w_o = oracle.loss_weights(c.mask, c.B, c.L, "token")
    args = dict(z=z64, ids=c.ids, old_logp=old.astype(np.float64), ref_logp=None,
                adv=adv.cpu().numpy().astype(np.float64), mask=c.mask, B=c.B, L=c.L,
                level="token", **kw)
    o = oracle.grpo_forward(**args)
    _, g, zero_o = oracle.grpo_backward(dloss=w_o, fwd=o, **args)
    zero = zr.cpu().numpy().astype(bool)
    assert np.array_equal(zero, zero_o.astype(bool))
    assert zero[:4 * c.L].all()          # the all-equal group
    assert (bits(dz)[zero] == 0).all()


def test_mask_entries_are_boolean():
    """Nonzero mask entries count as 1: a 0/2 mask gives bit-identical
    sequence-level forward and backward and loss weights."""
    lib = require_gpu()
    c = fill_dloss(synth.grpo_sequence_case(with_logits=False, B=4, L=64, V=2048))
    say("mask 0/2 == mask 0/1: sequence level B4 L64 V2048, weights")
    rng = np.random.default_rng(51)
    zb = synth.f32_to_bf16_bits((rng.standard_normal((c.N, c.V)) * 2).astype(np.float32))
    z = logits_to_dev(zb, "bf16")
    mask = (rng.random(c.N) < 0.8).astype(np.uint8)
    old = (rng.standard_normal(c.N) * 0.3 - 7.0).astype(np.float32)
    kw = dict(temperature=1.0, beta=0.0, eps_low=0.2, eps_high=0.28, level="sequence")
    res = []
    for m in (mask, mask * 2):
        w = lib.grpo_loss_weights(dev(m), c.B, c.L, "sequence")
        fwd = lib.grpo_logits_fwd(z, dev(c.ids), dev(old), dev(c.adv), c.B, c.L, mask=dev(m), **kw)
        dz, zr = lib.grpo_logits_bwd(z, dev(c.ids), dev(old), dev(c.adv), c.B, c.L, fwd["logp"],
                                     fwd["lse"], w, mask=dev(m), seq_ratio=fwd["seq_ratio"], **kw)
        torch.cuda.synchronize()
        res.append((bits(w), bits(fwd["loss"]), bits(fwd["seq_ratio"]), bits(dz), zr.cpu().numpy()))
    for x, y in zip(*res):
        assert np.array_equal(x, y)
