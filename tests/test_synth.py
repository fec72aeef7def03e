"""Seeded input generators: determinism, stated structure, bf16 rounding."""
import numpy as np
import torch

import synth
from case_weights import fill_dloss


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65504.0, 1e-40],
                                 np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_blocked_matrix_rows_and_determinism():
    s = synth.streams(0)
    full = synth.normal_matrix(s["logits"], 1000, 37, 2.0, True)
    again = synth.normal_matrix(synth.streams(0)["logits"], 1000, 37, 2.0, True)
    assert np.array_equal(full, again)
    rows = np.array([999, 0, 257, 256, 511, 3])
    part = synth.normal_matrix(s["logits"], 1000, 37, 2.0, True, rows=rows)
    assert np.array_equal(part, full[rows])
    other = synth.normal_matrix(synth.streams(1)["logits"], 1000, 37, 2.0, True)
    assert not np.array_equal(full, other)


def test_tiny_case_structure():
    c = fill_dloss(synth.tiny_case("a"))
    assert c.logits.shape == (32, 1024) and c.logits.dtype == np.float32
    assert c.adv[1] == 0.0 and c.adv[0] != 0.0
    assert c.mask.all() and c.ids.min() >= 0 and c.ids.max() < 1024
    assert abs(c.logits.std() - 2.0) < 0.05
    assert fill_dloss(synth.tiny_case("c")).ref_noise is None
    assert fill_dloss(synth.tiny_case("b")).beta == 0.0


def test_token_case_structure():
    c = fill_dloss(synth.grpo_token_case(with_logits=False))
    assert c.N == 2048 and (c.adv == 0).sum() == 2
    m = c.mask.reshape(4, 512)
    lens = m.sum(axis=1)
    assert (lens >= 256).all() and (lens <= 512).all()
    for b in range(4):   # trailing padding
        assert m[b, :lens[b]].all() and not m[b, lens[b]:].any()
    np.testing.assert_allclose(c.dloss.sum(), 1.0, rtol=1e-6)
    assert c.ref_noise is None
    assert fill_dloss(synth.grpo_token_case(with_logits=False, with_ref=True)).ref_noise is not None


def test_sequence_case_structure():
    c = fill_dloss(synth.grpo_sequence_case(with_logits=False))
    assert (c.adv == 0).sum() == 2 and c.beta == 0.0 and c.level == "sequence"
    per_seq = c.old_noise.reshape(8, 1024)
    assert (per_seq == per_seq[:, :1]).all()   # one perturbation per sequence


def test_row_case_peak_rows():
    c = synth.row_case(N=600, V=500)
    rows = np.array([5, 300, 599])
    assert np.array_equal(c.logits_rows(rows), c.logits[rows])
    z = synth.bf16_bits_to_f32(c.logits)
    at_peak = z[np.arange(600), c.peak_cols]
    assert abs(at_peak.mean() - 8.0) < 0.5 and abs(z.mean()) < 0.05


def test_fused_case_structure():
    c = fill_dloss(synth.fused_case(B=4, L=8, H=16, V=64))
    assert c.hidden.shape == (32, 16) and c.weight.shape == (64, 16)
    assert (c.adv == 0).sum() == 2
    lens = c.mask.reshape(4, 8).sum(axis=1)
    assert (lens >= 4).all() and (lens <= 8).all()


def test_stored_tiny_logp_is_the_oracles():
    """The stored logp / lse of the tiny case (written by
    tests/golden/make_oracle_logp.py from the oracle alone) equal the
    oracle's on the generator's current inputs."""
    import oracle
    c = fill_dloss(synth.tiny_case("a"))
    lp = synth.load_stored_logp("tiny", c.logits[synth.stored_check_rows("tiny")])
    lse = synth.load_stored_lse("tiny")
    want_lp, want_lse = oracle.selective_log_softmax(c.logits.astype(np.float64), c.ids,
                                                     c.temperature)
    assert np.array_equal(lp, want_lp) and np.array_equal(lse, want_lse)
