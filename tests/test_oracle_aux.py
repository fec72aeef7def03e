"""Pins of the oracle's steps either side of the row pass: entropy backward,
group-relative advantages and loss-reduction weights (CPU only).

Each is checked against something other than its own formula: finite
differences of the entropy, a two-class closed form, hand-computed values,
invariants of the definitions, brute-force loops."""
import math

import numpy as np
import pytest

import oracle


# -- entropy backward ---------------------------------------------------------
def _entropy_objective(z, g, T):
    return float((g * oracle.entropy_from_logits(z, T)).sum())


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_entropy_bwd_matches_central_differences(T):
    rng = np.random.default_rng(11)
    z = rng.standard_normal((3, 7)) * 1.5
    g = rng.standard_normal(3)
    dz = oracle.entropy_from_logits_bwd(z, g, T)
    h = 1e-6
    num = np.zeros_like(z)
    for r in range(z.shape[0]):
        for j in range(z.shape[1]):
            zp = z.copy(); zp[r, j] += h
            zm = z.copy(); zm[r, j] -= h
            num[r, j] = (_entropy_objective(zp, g, T) - _entropy_objective(zm, g, T)) / (2 * h)
    np.testing.assert_allclose(dz, num, rtol=1e-6, atol=1e-9)


def test_entropy_bwd_two_class_closed_form():
    """z = [a, 0], T = 1: H(a) = binary entropy of sigma(a), dH/da = -a s (1 - s)."""
    for a in (-3.0, -0.4, 0.0, 0.9, 2.5):
        s = 1.0 / (1.0 + math.exp(-a))
        dz = oracle.entropy_from_logits_bwd(np.array([[a, 0.0]]), np.array([1.0]))
        assert abs(dz[0, 0] - (-a * s * (1 - s))) <= 1e-14
        assert abs(dz[0, 1] + dz[0, 0]) <= 1e-14


def test_entropy_bwd_rows_sum_to_zero_and_uniform_rows_vanish():
    rng = np.random.default_rng(12)
    z = rng.standard_normal((5, 33)) * 2
    z[2] = 0.75  # uniform row: H = log V is stationary
    g = rng.standard_normal(5)
    g[4] = 0.0
    dz = oracle.entropy_from_logits_bwd(z, g, 0.9)
    assert np.abs(dz.sum(axis=1)).max() <= 1e-14
    assert np.abs(dz[2]).max() <= 1e-15
    assert (dz[4] == 0.0).all()


# -- group-relative advantages ------------------------------------------------
def test_group_advantages_hand_example():
    """[1, 0, 0, 1]: mean 1/2, sample std sqrt(1/3); A = +-(1/2) / (sqrt(1/3) + 1e-4)."""
    a = oracle.group_advantages(np.array([1.0, 0.0, 0.0, 1.0]), 4)
    want = 0.5 / (math.sqrt(1.0 / 3.0) + 1e-4)
    np.testing.assert_allclose(a, [want, -want, -want, want], rtol=0, atol=1e-15)
    b = oracle.group_advantages(np.array([3.0, 1.0]), 2, eps=0.0, scale=False)
    np.testing.assert_array_equal(b, [1.0, -1.0])


def test_group_advantages_invariants():
    rng = np.random.default_rng(13)
    G = 8
    r = rng.standard_normal(6 * G)
    r[2 * G:3 * G] = 0.1          # all equal: exactly zero (the zero-advantage case)
    a = oracle.group_advantages(r, G, eps=0.0).reshape(-1, G)
    assert (a[2] == 0.0).all()
    keep = [0, 1, 3, 4, 5]
    assert np.abs(a[keep].sum(axis=1)).max() <= 1e-13
    np.testing.assert_allclose(a[keep].std(axis=1, ddof=1), 1.0, rtol=1e-12)
    # binary rewards: groups of all-0 or all-1 give zero advantage
    rb = np.array([0, 0, 0, 0, 1, 1, 1, 1, 1, 0, 0, 0], dtype=np.float64)
    ab = oracle.group_advantages(rb, 4)
    assert (ab[:8] == 0.0).all() and (ab[8:] != 0.0).all()
    # groups of one have no spread
    assert (oracle.group_advantages(np.array([2.0, -1.0]), 1) == 0.0).all()


# -- loss-reduction weights -----------------------------------------------------
def _mask(B, L, rng):
    lengths = rng.integers(0, L + 1, size=B)
    lengths[0] = L
    return (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8).reshape(-1), lengths


@pytest.mark.parametrize("reduction", ["token", "sequence", "constant"])
def test_loss_weights_equal_brute_force_reduction(reduction):
    rng = np.random.default_rng(14)
    B, L = 5, 9
    mask, lengths = _mask(B, L, rng)
    lengths[1] = 0
    mask = (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8).reshape(-1)
    loss = rng.standard_normal(B * L)
    w = oracle.loss_weights(mask, B, L, reduction)
    if reduction == "token":
        tot, n = 0.0, 0
        for b in range(B):
            for t in range(L):
                if mask[b * L + t]:
                    tot += loss[b * L + t]; n += 1
        want = tot / n
    elif reduction == "sequence":
        want = 0.0
        for b in range(B):
            if lengths[b]:
                want += sum(loss[b * L + t] for t in range(lengths[b])) / lengths[b]
        want /= B
    else:
        want = sum(loss[i] for i in range(B * L) if mask[i]) / (B * L)
    assert abs(float((w * loss).sum()) - want) <= 1e-13
    assert (w[mask == 0] == 0.0).all()


def test_loss_weights_closed_sums():
    B, L = 4, 6
    mask = np.ones(B * L, dtype=np.uint8)
    mask[L:2 * L] = 0
    assert abs(oracle.loss_weights(mask, B, L, "token").sum() - 1.0) <= 1e-15
    ws = oracle.loss_weights(mask, B, L, "sequence").reshape(B, L).sum(axis=1)
    np.testing.assert_allclose(ws, [0.25, 0.0, 0.25, 0.25], atol=1e-15)
    assert (oracle.loss_weights(None, B, L, "constant") == 1.0 / (B * L)).all()
    assert (oracle.loss_weights(np.zeros(B * L), B, L, "token") == 0.0).all()


def test_mask_entries_are_boolean():
    """A completion mask's nonzero entries count as 1 (a 0/2 mask is the 0/1 mask)."""
    rng = np.random.default_rng(15)
    B, L = 3, 7
    mask = (rng.random(B * L) < 0.7).astype(np.uint8)
    for red in ("token", "sequence", "constant"):
        np.testing.assert_array_equal(oracle.loss_weights(mask * 2, B, L, red),
                                      oracle.loss_weights(mask, B, L, red))
    z = rng.standard_normal((B * L, 11))
    ids = rng.integers(0, 11, B * L)
    lp, _ = oracle.selective_log_softmax(z, ids)
    old = lp + rng.standard_normal(B * L) * 0.3
    adv = rng.standard_normal(B)
    args = dict(z=z, ids=ids, old_logp=old, ref_logp=None, adv=adv, B=B, L=L, temperature=1.0,
                beta=0.0, eps_low=0.2, eps_high=0.2, level="sequence")
    a = oracle.grpo_forward(mask=mask, **args)
    b = oracle.grpo_forward(mask=mask * 2, **args)
    for k in ("loss", "seq_ratio"):
        np.testing.assert_array_equal(a[k], b[k])
