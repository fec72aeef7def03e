"""Calls whose grids pass one dispatch's 32-bit work-item count.

A dispatch packet holds each grid dimension in work-items as a 32-bit
number, so the library cuts its per-row launches into slices of whole
workgroups.  V = 8 bf16 (one 16-byte vector per row) takes the smallest
launch shapes: 64 lanes per row in the forward and the single pass
(67108863 rows per launch), 256 in the backward, the selective and entropy
backwards (16777215 rows per launch), the sequence epilogue and the loss
weights (16777215 sequences per launch).  Just over 2^26 rows therefore need
two forward launches and five backward ones.

Inputs are seeded draws on the device (torch's generator): logits N(0, 2^2)
(the token-level workload's spread), ids uniform, old_logp = -ln 8 +
N(0, 0.3^2) and ref_logp = -ln 8 + N(0, 0.1^2) around the uniform row's
logp (ratios on both sides of the clip bounds), advantages N(0, 1) with
every fourth 0, 10% of tokens masked, the plain sum's weights (dloss = the
mask), and for the selective and entropy backwards N(0, 1) upstream
gradients with every fifth 0.

Checks: every output element of every row written (the NaN and 7 sentinels
gone), exact +0.0 rows where zero_row says, no invalid-id count; and the
whole sequences around every slice boundary, the first and the last and 32
drawn at random, against the oracle with the bars of test_rows_gpu.py and
test_rows_sweep_gpu.py."""
import math
import types

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (GrpoInputs, assert_bf16_dz, assert_rel, dev_to_f64, require_gpu, say)
from test_aux_gpu import _entropy_bound
from test_rows_gpu import check_backward, check_forward, oracle_expectations

pytestmark = pytest.mark.gpu

V = 8
ITEMS = 2 ** 32 - 1
FWD_STEP = ITEMS // 64    # rows per forward / single-pass launch
BWD_STEP = ITEMS // 256   # rows per backward launch; sequences per epilogue launch
T, EPS_LOW, EPS_HIGH = 0.9, 0.2, 0.28


def _draw(B, L, seed, V=V):
    g = torch.Generator(device="cuda").manual_seed(seed)
    N = B * L
    dv = dict(device="cuda", generator=g)
    lu = -math.log(V)
    d = dict(z=(torch.randn(N, V, **dv) * 2.0).to(torch.bfloat16),
             ids=torch.randint(0, V, (N,), **dv),
             old=lu + 0.3 * torch.randn(N, **dv),
             ref=lu + 0.1 * torch.randn(N, **dv),
             adv=torch.randn(B, **dv),
             mask=(torch.rand(N, **dv) >= 0.1).to(torch.uint8),
             grad=torch.randn(N, **dv))
    d["adv"][::4] = 0.0
    d["grad"][::5] = 0.0
    d["dloss"] = d["mask"].float()
    return d


def _sentinel(n, dtype=torch.float32, shape=None):
    fill = 7 if dtype == torch.uint8 else float("nan")
    return torch.full(shape or (n,), fill, dtype=dtype, device="cuda")


def _all_written(name, t):
    if t.dtype == torch.uint8:
        assert bool(((t == 0) | (t == 1)).all()), f"{name}: an element was not written"
    else:
        assert not bool(torch.isnan(t).any()), f"{name}: an element was not written"


def _zero_rows_exact(name, dz, zr):
    rows = dz.view(torch.int16)[zr.bool()]
    assert bool((rows == 0).all()), f"{name}: a zero row is not +0.0"


def _sample(B, L, rows_at, seqs_at, seed):
    """Whole sequences around the given row and sequence indexes, the first
    and the last sequence and 32 drawn at random (sorted, unique)."""
    N = B * L
    rng = np.random.default_rng(seed)
    rows = {0, N - 1}
    for r in rows_at:
        rows.update(range(max(0, r - 3), min(N, r + 3)))
    rows.update(rng.integers(0, N, 32).tolist())
    seqs = {r // L for r in rows}
    for b in seqs_at:
        seqs.update(range(max(0, b - 2), min(B, b + 2)))
    return np.array(sorted(seqs), dtype=np.int64)


def _sub_inputs(d, seqs, L, level, beta):
    """The sampled sequences as an oracle case (host arrays) and their row index."""
    rows = (seqs[:, None] * L + np.arange(L)[None, :]).reshape(-1)
    ri = torch.from_numpy(rows).cuda()
    si = torch.from_numpy(seqs).cuda()
    host = lambda t, i: t.index_select(0, i).cpu().numpy()
    z_bits = d["z"].index_select(0, ri).view(torch.int16).cpu().numpy().view(np.uint16)
    c = types.SimpleNamespace(
        B=len(seqs), L=L, N=len(rows), V=d["z"].shape[1], level=level, beta=beta, temperature=T,
        eps_low=EPS_LOW, eps_high=EPS_HIGH, ids=host(d["ids"], ri), adv=host(d["adv"], si),
        mask=host(d["mask"], ri), dloss=host(d["dloss"], ri))
    inp = GrpoInputs.__new__(GrpoInputs)
    inp.case, inp.old, inp.ref = c, host(d["old"], ri), host(d["ref"], ri)
    return c, inp, oracle.decode_bf16(z_bits), ri, si


def _grpo_outputs(N, B, level, with_gathered=True):
    o = dict(loss=_sentinel(N), logp=_sentinel(N), lse=_sentinel(N), entropy=_sentinel(N),
             kl=_sentinel(N), is_clipped=_sentinel(N, torch.uint8))
    if with_gathered:
        o["gathered"] = _sentinel(N)
    if level == "sequence":
        o["seq_ratio"] = _sentinel(B)
    return o


def _pick(outs, ri, si):
    return {k: (v.index_select(0, si) if k == "seq_ratio" else v.index_select(0, ri))
            for k, v in outs.items()}


def _entropy_selective(lib, d, N):
    """entropy_from_logits, selective_log_softmax and both backwards on the
    whole of d, into sentinel-filled outputs; the backwards take the
    forwards' lse and H."""
    V_ = d["z"].shape[1]
    H = lib.entropy_from_logits(d["z"], T, out=_sentinel(N))
    lp, lse = lib.selective_log_softmax(d["z"], d["ids"], T, out=_sentinel(N), lse=_sentinel(N))
    sdz = lib.selective_log_softmax_bwd(d["z"], d["ids"], lse, d["grad"], T,
                                        dlogits=_sentinel(N, torch.bfloat16, (N, V_)))
    edz = lib.entropy_from_logits_bwd(d["z"], lse, H, d["grad"], T,
                                      dlogits=_sentinel(N, torch.bfloat16, (N, V_)))
    return H, lp, lse, sdz, edz


def _check_entropy_selective(d, c, z64, ri, H, lp, lse, sdz, edz):
    gs = d["grad"].index_select(0, ri).cpu().numpy()
    lp_o, lse_o = oracle.selective_log_softmax(z64, c.ids, T)
    H_o = oracle.entropy_from_logits(z64, T)
    assert_rel(H.index_select(0, ri).cpu().numpy(), H_o, "entropy")
    assert_rel(lp.index_select(0, ri).cpu().numpy(), lp_o, "selective logp")
    assert_rel(lse.index_select(0, ri).cpu().numpy(), lse_o, "selective lse")
    g64 = gs.astype(np.float64)
    want = oracle.selective_log_softmax_bwd(z64, c.ids, g64, T)
    assert_bf16_dz(dev_to_f64(sdz.index_select(0, ri)), want, "selective backward")
    # the backwards take the library's lse and H, which carry the forwards'
    # bars (asserted just above): their effect on dz_j = -(g/T) p_j (log p_j
    # + H) is at most |g/T| p_j (d_lse (1 + |log p_j + H|) + d_H)
    wantH = oracle.entropy_from_logits_bwd(z64, g64, T)
    logp = z64 / T - lse_o[:, None]
    p = np.exp(logp)
    d_lse, d_H = 1e-5 * np.abs(lse_o) + 1e-6, 1e-5 * np.abs(H_o) + 1e-6
    tolH = (1e-5 + 2.0 ** -8) * np.abs(wantH) + _entropy_bound(z64, T, gs, lse_o, H_o) + \
        (np.abs(g64) / T)[:, None] * p * (d_lse[:, None] * (1 + np.abs(logp + H_o[:, None]))
                                          + d_H[:, None]) + 1e-30
    errH = np.abs(dev_to_f64(edz.index_select(0, ri)) - wantH)
    assert (errH <= tolH).all(), f"entropy backward: max err {errH.max()}"
    say("  entropy and selective log-softmax, forward and backward, match the oracle")


def test_token_level_past_one_dispatch():
    lib = require_gpu()
    L = 7
    B = FWD_STEP // L + 600            # 67112969 rows
    N = B * L
    beta = 0.04
    assert N > FWD_STEP and N > 4 * BWD_STEP
    say(f"token level past one dispatch: B={B} L={L} ({N} rows) V={V} bf16; "
        f"{-(-N // FWD_STEP)} forward, {-(-N // BWD_STEP)} backward launches")
    d = _draw(B, L, seed=11)
    kw = dict(temperature=T, beta=beta, eps_low=EPS_LOW, eps_high=EPS_HIGH)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fwd = lib.grpo_logits_fwd(d["z"], d["ids"], d["old"], d["adv"], B, L, ref_logp=d["ref"],
                              mask=d["mask"], err_count=err, out=_grpo_outputs(N, B, "token"),
                              **kw)
    dz, zr = lib.grpo_logits_bwd(d["z"], d["ids"], d["old"], d["adv"], B, L, fwd["logp"],
                                 fwd["lse"], d["dloss"], ref_logp=d["ref"], mask=d["mask"],
                                 dlogits=_sentinel(N, torch.bfloat16, (N, V)),
                                 zero_row=_sentinel(N, torch.uint8), **kw)
    err1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    one, dz1, zr1 = lib.grpo_logits_fwd_bwd(
        d["z"], d["ids"], d["old"], d["adv"], B, L, d["dloss"], ref_logp=d["ref"],
        mask=d["mask"], dlogits=_sentinel(N, torch.bfloat16, (N, V)),
        zero_row=_sentinel(N, torch.uint8), err_count=err1,
        out=_grpo_outputs(N, B, "token", with_gathered=False), **kw)
    H, lp, lse, sdz, edz = _entropy_selective(lib, d, N)
    torch.cuda.synchronize()

    for name, t in list(fwd.items()) + [("dz", dz), ("zero_row", zr)] + \
            [(f"single {k}", v) for k, v in one.items()] + \
            [("single dz", dz1), ("single zero_row", zr1), ("entropy", H), ("selective logp", lp),
             ("selective lse", lse), ("selective dz", sdz), ("entropy dz", edz)]:
        _all_written(name, t)
    _zero_rows_exact("dz", dz, zr)
    _zero_rows_exact("single dz", dz1, zr1)
    _zero_rows_exact("selective dz", sdz, d["grad"] == 0)
    _zero_rows_exact("entropy dz", edz, d["grad"] == 0)
    assert int(err.item()) == 0 and int(err1.item()) == 0
    say(f"  every row written; zero rows: {int(zr.sum())} of {N}")

    bounds = [FWD_STEP] + [k * BWD_STEP for k in range(1, -(-N // BWD_STEP))]
    seqs = _sample(B, L, bounds, [], seed=12)
    c, inp, z64, ri, si = _sub_inputs(d, seqs, L, "token", beta)
    say(f"  oracle on {len(seqs)} sequences around the slice boundaries {bounds}")
    for what, outs, dzx, zrx in (("two-pass", fwd, dz, zr), ("single pass", one, dz1, zr1)):
        got = _pick(outs, ri, si)
        got["err_count"] = err
        o, g = oracle_expectations(inp, z64, got)
        check_forward(c, o, got, ref=inp.ref)
        check_backward(c, o, g, dzx.index_select(0, ri), zrx.index_select(0, ri), z64, inp)
        say(f"  {what}: forward and backward match the oracle")

    _check_entropy_selective(d, c, z64, ri, H, lp, lse, sdz, edz)


def test_sequence_level_past_one_dispatch():
    lib = require_gpu()
    L = 4
    B = BWD_STEP + 85                  # 16777300 sequences, 67109200 rows
    N = B * L
    beta = 0.0
    assert N > FWD_STEP and B > BWD_STEP
    say(f"sequence level past one dispatch: B={B} L={L} ({N} rows) V={V} bf16; "
        f"{-(-B // BWD_STEP)} epilogue and loss-weight launches")
    d = _draw(B, L, seed=21)
    kw = dict(temperature=T, beta=beta, eps_low=EPS_LOW, eps_high=EPS_HIGH, level="sequence")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fwd = lib.grpo_logits_fwd(d["z"], d["ids"], d["old"], d["adv"], B, L, mask=d["mask"],
                              err_count=err, out=_grpo_outputs(N, B, "sequence"), **kw)
    dz, zr = lib.grpo_logits_bwd(d["z"], d["ids"], d["old"], d["adv"], B, L, fwd["logp"],
                                 fwd["lse"], d["dloss"], mask=d["mask"],
                                 seq_ratio=fwd["seq_ratio"],
                                 dlogits=_sentinel(N, torch.bfloat16, (N, V)),
                                 zero_row=_sentinel(N, torch.uint8), **kw)
    w = lib.grpo_loss_weights(d["mask"], B, L, "sequence", dloss=_sentinel(N))
    torch.cuda.synchronize()
    for name, t in list(fwd.items()) + [("dz", dz), ("zero_row", zr), ("weights", w)]:
        _all_written(name, t)
    _zero_rows_exact("dz", dz, zr)
    assert int(err.item()) == 0
    say(f"  every row written; zero rows: {int(zr.sum())} of {N}")

    bounds = [FWD_STEP] + [k * BWD_STEP for k in range(1, -(-N // BWD_STEP))]
    seqs = _sample(B, L, bounds, [BWD_STEP], seed=22)
    c, inp, z64, ri, si = _sub_inputs(d, seqs, L, "sequence", beta)
    inp.ref = None
    say(f"  oracle on {len(seqs)} sequences around the slice boundaries {bounds} "
        f"and sequence {BWD_STEP}")
    got = _pick(fwd, ri, si)
    got["err_count"] = err
    o, g = oracle_expectations(inp, z64, got)
    check_forward(c, o, got, ref=None)
    check_backward(c, o, g, dz.index_select(0, ri), zr.index_select(0, ri), z64, inp)
    # the sequence mean's weights: 1 / (n_b B) on every kept token (rounded
    # once to fp32 from the exact value), 0 on masked ones
    ws = w.index_select(0, ri).cpu().numpy().astype(np.float64).reshape(-1, L)
    m = c.mask.reshape(-1, L) != 0
    n_b = np.maximum(m.sum(1), 1)[:, None]
    assert (ws[~m] == 0.0).all()
    assert (np.abs(ws * n_b * B - 1.0)[m] <= 2.0 ** -23).all()
    say("  forward, backward and the sequence-mean weights match the oracle")


def test_longest_rows():
    """Two rows of V = 2^26 bf16 (128 MB each), the longest the library
    accepts: the forward streams each row with one 1024-lane workgroup, the
    backward splits each into 16384 chunks of 512 vectors (the entropy
    backward into 2048 of 4096), and the single pass, whose rows must fit in
    registers, runs as forward then backward.  Row 0 samples the last column
    and has weight 0 (a zero row over all of its chunks), row 1 the first."""
    lib = require_gpu()
    Vmax = 1 << 26
    B, L = 2, 1
    N = B * L
    beta = 0.04
    say(f"longest rows: {N} rows of V = 2^26 bf16 ({N * Vmax * 2 >> 20} MiB)")
    d = _draw(B, L, seed=31, V=Vmax)
    d["ids"][0], d["ids"][1] = Vmax - 1, 0
    d["mask"][:] = 1
    d["dloss"][:] = torch.tensor([0.0, 1.0], device="cuda")
    d["grad"][:] = torch.tensor([0.0, 0.7], device="cuda")
    kw = dict(temperature=T, beta=beta, eps_low=EPS_LOW, eps_high=EPS_HIGH)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fwd = lib.grpo_logits_fwd(d["z"], d["ids"], d["old"], d["adv"], B, L, ref_logp=d["ref"],
                              mask=d["mask"], err_count=err, out=_grpo_outputs(N, B, "token"),
                              **kw)
    dz, zr = lib.grpo_logits_bwd(d["z"], d["ids"], d["old"], d["adv"], B, L, fwd["logp"],
                                 fwd["lse"], d["dloss"], ref_logp=d["ref"], mask=d["mask"],
                                 dlogits=_sentinel(N, torch.bfloat16, (N, Vmax)),
                                 zero_row=_sentinel(N, torch.uint8), **kw)
    err1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    one, dz1, zr1 = lib.grpo_logits_fwd_bwd(
        d["z"], d["ids"], d["old"], d["adv"], B, L, d["dloss"], ref_logp=d["ref"],
        mask=d["mask"], dlogits=_sentinel(N, torch.bfloat16, (N, Vmax)),
        zero_row=_sentinel(N, torch.uint8), err_count=err1,
        out=_grpo_outputs(N, B, "token", with_gathered=False), **kw)
    H, lp, lse, sdz, edz = _entropy_selective(lib, d, N)
    torch.cuda.synchronize()
    for name, t in list(fwd.items()) + [("dz", dz), ("zero_row", zr)] + \
            [(f"single {k}", v) for k, v in one.items()] + \
            [("single dz", dz1), ("single zero_row", zr1), ("entropy", H), ("selective logp", lp),
             ("selective lse", lse), ("selective dz", sdz), ("entropy dz", edz)]:
        _all_written(name, t)
    assert zr.tolist() == [1, 0] and zr1.tolist() == [1, 0]
    assert int(err.item()) == 0 and int(err1.item()) == 0

    c, inp, z64, ri, si = _sub_inputs(d, np.arange(B, dtype=np.int64), L, "token", beta)
    for what, outs, dzx, zrx in (("two-pass", fwd, dz, zr), ("single pass", one, dz1, zr1)):
        got = _pick(outs, ri, si)
        got["err_count"] = err
        o, g = oracle_expectations(inp, z64, got)
        check_forward(c, o, got, ref=inp.ref)
        check_backward(c, o, g, dzx, zrx, z64, inp)
        say(f"  {what}: forward and backward match the oracle")
    _check_entropy_selective(d, c, z64, ri, H, lp, lse, sdz, edz)


def test_fused_chunk_past_one_dispatch():
    """The chunked fused-linear loss on 16778216 one-token sequences (H = 64,
    V = 8, every row weighted): the row gather (one 256-lane workgroup per
    kept row) takes two launches, the boundary at compact row 16777215 (every
    row is kept, so compact row i is row i).  grad_hidden of the rows around
    the boundary, the first, the last and 16 drawn at random against the
    oracle within the per-element bound of test_fused_gpu.py; every row of
    grad_hidden written; loss and grad_weight finite."""
    from test_fused_gpu import U, _assert_bound, _coef_error, _dz_error
    lib = require_gpu()
    H, Vf, beta = 64, 8, 0.04
    R = BWD_STEP + 1001
    say(f"fused chunk past one dispatch: {R} rows (one token each), H={H} V={Vf}; "
        f"{-(-R // BWD_STEP)} gather launches")
    g = torch.Generator(device="cuda").manual_seed(41)
    dv = dict(device="cuda", generator=g)
    lu = -math.log(Vf)
    h = torch.randn(R, H, **dv).to(torch.bfloat16)
    W = (torch.randn(Vf, H, **dv) * 0.25).to(torch.bfloat16)
    ids = torch.randint(0, Vf, (R,), **dv)
    old = lu + 0.3 * torch.randn(R, **dv)
    ref = lu + 0.1 * torch.randn(R, **dv)
    adv = torch.randn(R, **dv)
    adv[::4] = 0.0
    dloss = torch.ones(R, device="cuda")
    gh = _sentinel(R * H).view(R, H)
    loss, gh, gW = lib.fused_linear_grpo_chunk(h, W, ids, old, adv, None, dloss, R, 1,
                                               ref_logp=ref, temperature=T, beta=beta,
                                               eps_low=EPS_LOW, eps_high=EPS_HIGH,
                                               grad_hidden=gh)
    torch.cuda.synchronize()
    _all_written("grad_hidden", gh)
    assert bool(torch.isfinite(loss).all()) and bool(torch.isfinite(gW).all())

    rng = np.random.default_rng(42)
    rows = np.unique(np.concatenate([np.arange(BWD_STEP - 4, BWD_STEP + 4), [0, R - 1],
                                     rng.integers(0, R, 16)])).astype(np.int64)
    ri = torch.from_numpy(rows).cuda()
    host = lambda t: t.index_select(0, ri).cpu().numpy()
    hb = h.index_select(0, ri).view(torch.int16).cpu().numpy().view(np.uint16)
    hs = oracle.decode_bf16(hb)
    W64 = oracle.decode_bf16(W.view(torch.int16).cpu().numpy().view(np.uint16))
    n = len(rows)
    ids_s, old_s, ref_s = host(ids), host(old).astype(np.float64), host(ref).astype(np.float64)
    adv_s, w_s = host(adv), host(dloss)
    z = hs @ W64.T
    fwd = oracle.grpo_forward(z, ids_s, old_s, ref_s, adv_s, None, n, 1, T, beta, EPS_LOW,
                              EPS_HIGH)
    gs = oracle.grpo_dlogp(fwd, ref_s, adv_s, None, w_s, n, 1, beta)
    e_g = _coef_error(fwd["logp"], fwd["ratio"], fwd["is_clipped"],
                      adv_s.astype(np.float64), ref_s, w_s.astype(np.float64), beta)
    aW = np.abs(W64)
    zeta = 2 * H * U * (np.abs(hs) @ aW.T)
    onehot = np.zeros_like(z)
    onehot[np.arange(n), ids_s] = 1.0
    dz, E = _dz_error(z, zeta, fwd["lse"], gs, e_g, onehot, T)
    want = dz @ W64
    bound = E @ aW + 2 * (Vf + 1) * U * ((np.abs(dz) + E) @ aW)
    worst = _assert_bound(host(gh), want, bound, "grad_hidden")
    say(f"  {n} rows of grad_hidden around compact row {BWD_STEP} within the bound "
        f"(largest error / bound {worst:.3f})")
