"""GPU parity of the bf16 MFMA GEMM and of the chunked fused-linear GRPO loss.

GEMM: against float64 products of the same bf16 values; the bound is the
fp32 accumulation error, |err| <= 2 K 2^-24 sum_k |a_mk b_kn| (+ the same for
the accumulated C).
Fused linear: loss within 1e-5 relative (row statistics and target logit
from the logits product's fp32 accumulators).  grad_hidden and grad_weight:
every element within a bound derived from the chunk's two bf16 roundings and
the fp32 accumulations (the backward's softmax reads z rounded to bf16, and
dz is rounded to bf16 before the two products).  With u = 2^-24,
p = softmax(z/T) and the oracle's dz, g, lse, logp, the error of one dz
element is at most
    E = |g/T| p ((2^-8 |z| + zeta) / T + e_lse + 2^-22 (1 + |z|/T))
        + 2^-8 |dz| + (e_g / T) |onehot - p|
where zeta = 2 H u sum_k |h_k W_k| (the logits' accumulation), e_lse =
1e-5 |lse| + 1e-6 and e_logp = 1e-5 |logp| + 1e-6 (the forward's bar) and
e_g = (|ratio A| [not clipped] + beta e^{ref - logp}) |dloss| e_logp (the
coefficient's derivative in logp times that error); 2^-8 is twice bf16's
half-ulp, 2^-22 covers the exponent's fp32 arithmetic.  Then
    |grad_hidden[r,k] err| <= sum_j E_rj |W_jk| + 2 (V + 1) u sum_j (|dz| + E)_rj |W_jk|
    |grad_weight[j,k] err| <= sum_r E_rj |h_rk| + 2 (N + chunks) u sum_r (|dz| + E)_rj |h_rk|
(accumulation over V, split-K partial sums included; over the rows of every
chunk plus one fp32 add per chunk).  Being a worst case over |.|, the bound
is loose where a gradient cancels across rows; the relative Frobenius error
(1e-2 per tensor, and per sampled row / vocabulary entry at the workload's
temperature) is kept beside it.  Rows of grad_hidden whose dlogp is 0 are
exactly 0.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from case_weights import fill_dloss
from gpu_common import dev, require_gpu, say

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    bits = synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))
    return bits, oracle.decode_bf16(bits)


def _t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("a_layout,b_layout", [(0, 0), (0, 1), (1, 1), (1, 0)])
@pytest.mark.parametrize("M,N,K", [(128, 128, 32), (200, 264, 96), (520, 392, 1064), (8, 16, 8),
                                   (4000, 7880, 136), (2056, 14344, 72), (4096, 8192, 200),
                                   (2056, 14344, 128), (4104, 8200, 192),
                                   (32776, 1032, 64), (32776, 1032, 72)])
def test_gemm_layouts(a_layout, b_layout, M, N, K):
    """The first four shapes take the 128 x 128 block tile; (4000, 7880, 136)
    has fewer than 512 tiles of 256 x 256 but at least 512 of 256 x 128, so a
    transposed operand takes the 256 x 128 tile (K-contiguous ones the
    128 x 128); the last six (>= 512 tiles of 256 x 256) take the pipelined
    256 x 256 x 64 tile in every layout: ragged in M, N and K (the masked
    loop), and ragged in M and N only with whole K steps (the unmasked loop,
    its loads clamped into the operands at the overhanging tiles).  The two
    with N = 1032 have 5 column tiles, so each XCD's run of tiles takes
    successive n for one m (the order of the fused path's gradient
    products)."""
    lib = require_gpu()
    say(f"gemm layouts a={a_layout} b={b_layout} M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a_bits, a = _bf16(rng, (M, K) if a_layout == 0 else (K, M))
    b_bits, b = _bf16(rng, (N, K) if b_layout == 0 else (K, N))
    A = a if a_layout == 0 else a.T
    Bm = b.T if b_layout == 0 else b
    ref = A @ Bm
    bound = 2 * K * 2.0 ** -24 * (np.abs(A) @ np.abs(Bm)) + 1e-30
    C = lib.grpo_gemm_bf16(_t(a_bits), _t(b_bits), a_layout=a_layout, b_layout=b_layout)
    torch.cuda.synchronize()
    err = np.abs(C.cpu().numpy() - ref)
    assert (err <= bound).all(), f"max err {err.max()} (bound {bound[err > bound][:3]})"
    # accumulate into an existing C
    C0 = rng.standard_normal((M, N)).astype(np.float32)
    C2 = lib.grpo_gemm_bf16(_t(a_bits), _t(b_bits), a_layout=a_layout, b_layout=b_layout,
                            C=dev(C0), accumulate=True)
    torch.cuda.synchronize()
    err2 = np.abs(C2.cpu().numpy() - (C0.astype(np.float64) + ref))
    assert (err2 <= bound + 2.0 ** -23 * np.abs(C0)).all()


@pytest.mark.parametrize("M,N,K,T", [(520, 1032, 136, 0.9), (300, 264, 64, 0.9), (40, 8, 8, 0.9),
                                     (4096, 8200, 136, 0.9), (520, 1032, 136, 0.05),
                                     (2056, 14344, 128, 0.9)])
def test_gemm_logits_mode(M, N, K, T):
    """The fused chunk's logits product alone (grpo_gemm_bf16_logits): against
    float64 products of the same bf16 values, z16 within the accumulation
    bound plus bf16 rounding, every partial's max within the bound, the merged
    log-sum-exp of z/T within 1e-5 relative plus the bound's effect, and the
    target logit within the bound (rows with an out-of-range id untouched).
    Where the fp32 store mode runs the same pipelined tile (>= 512 tiles:
    (4096, 8200, 136) and (2056, 14344, 128)) the results are exact against
    it: z16 is the correctly rounded fp32 C, zy and each max are entries of
    C.  N = 1032 and 264 leave 8 and 0 columns in the last 128-column
    half-tile, (40, 8, 8) is a single tile, and (2056, 14344, 128) overhangs
    M and N with whole K steps (the unmasked loop at the edge tiles).  At
    T = 0.05 each partial's sum must be referenced to its exact max for the
    merged log-sum-exp to meet its bar."""
    lib = require_gpu()
    say(f"gemm logits mode M={M} N={N} K={K} T={T}")
    rng = np.random.default_rng(M + N + K)
    a_bits, a = _bf16(rng, (M, K))
    b_bits, b = _bf16(rng, (N, K), 0.3)
    ids = rng.integers(0, N, M).astype(np.int64)
    ids[0] = -1
    ids[min(3, M - 1)] = N
    A, B = _t(a_bits), _t(b_bits)
    z16, stat, zy = lib.grpo_gemm_bf16_logits(A, B, dev(ids), temperature=T)
    C = lib.grpo_gemm_bf16(A, B)
    torch.cuda.synchronize()
    Z = a @ b.T
    bound = 2 * K * 2.0 ** -24 * (np.abs(a) @ np.abs(b).T) + 1e-30
    z16b = z16.view(torch.int16).cpu().numpy().view(np.uint16)
    zg = oracle.decode_bf16(z16b)
    assert (np.abs(zg - Z) <= bound + 2.0 ** -8 * (np.abs(Z) + bound)).all()  # bf16 unit roundoff 2^-8
    Cn = C.cpu().numpy()
    same_kernel = ((M + 255) // 256) * ((N + 255) // 256) >= 512
    if same_kernel:
        assert np.array_equal(z16b, synth.f32_to_bf16_bits(Cn))
    st = stat.cpu().numpy().astype(np.float64)
    P = lib.logits_partials(N)
    assert st.shape == (2, P, M)
    lse = np.full(M, -np.inf)
    for p in range(P):
        cols = np.arange(128 * p, min(128 * p + 128, N))
        if cols.size == 0:
            assert (st[0, p] == float(np.float32(-1e30))).all() and (st[1, p] == 0.0).all()
            continue
        m_ref = Z[:, cols].max(axis=1)
        mb = bound[:, cols].max(axis=1)
        assert (np.abs(st[0, p] - m_ref) <= mb).all()
        if same_kernel:
            assert np.array_equal(st[0, p].astype(np.float32), Cn[:, cols].max(axis=1))
        lse = np.logaddexp(lse, st[0, p] / T + np.log(st[1, p]))
    lse_ref = np.log(np.exp((Z - Z.max(axis=1, keepdims=True)) / T).sum(axis=1)) + Z.max(axis=1) / T
    tol = 1e-5 * np.abs(lse_ref) + 1e-6 + 2 * bound.max(axis=1) / T
    assert (np.abs(lse - lse_ref) <= tol).all()
    zyn = zy.cpu().numpy()
    ok = (ids >= 0) & (ids < N)
    r = np.flatnonzero(ok)
    assert (np.abs(zyn[r] - Z[r, ids[r]]) <= bound[r, ids[r]]).all()
    if same_kernel:
        assert np.array_equal(zyn[r], Cn[r, ids[r]])
    assert np.isnan(zyn[~ok]).all()


def _fused_inputs(case, logp_true):
    old = synth.add_noise_f32(logp_true, case.old_noise)
    ref = synth.add_noise_f32(logp_true, case.ref_noise)
    return old, ref


def _run_fused(lib, case, old, ref, chunk, stream=None):
    T = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
             eps_high=case.eps_high)
    h = _t(case.hidden)
    W = _t(case.weight)
    ids, old_t, ref_t, adv, mask, dl = (dev(case.ids), dev(old), dev(ref), dev(case.adv),
                                        dev(case.mask), dev(case.dloss))
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    gW = torch.zeros((case.V, case.H), dtype=torch.float32, device="cuda")
    gh = torch.empty((case.N, case.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.fused_linear_grpo_workspace_bytes(chunk * case.L, case.V, case.H),
                     dtype=torch.uint8, device="cuda")
    for b0 in range(0, case.B, chunk):
        nb = min(chunk, case.B - b0)
        rs = slice(b0 * case.L, (b0 + nb) * case.L)
        lib.fused_linear_grpo_chunk(h[rs], W, ids[rs], old_t[rs], adv[b0:b0 + nb], mask[rs],
                                    dl[rs], nb, case.L, ref_logp=ref_t[rs], loss_accum=loss,
                                    grad_hidden=gh[rs], grad_weight=gW, workspace=ws,
                                    stream=stream, **T)
    torch.cuda.synchronize()
    return float(loss.item()), gh.cpu().numpy(), gW


def _frob(got, want):
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


U = 2.0 ** -24


def _dz_error(z, zeta, lse, g, e_g, onehot, T):
    """Bound E on |dz_chunk - dz_exact| (module doc), with the oracle's dz;
    rows of z are the rows of g, lse, e_g (any subset of columns)."""
    p = np.exp(z / T - lse[:, None])
    dz = (g / T)[:, None] * (onehot - p)
    dz[g == 0.0] = 0.0
    E = (np.abs(g / T)[:, None] * p *
         ((2.0 ** -8 * np.abs(z) + zeta) / T + (1e-5 * np.abs(lse) + 1e-6)[:, None]
          + 2.0 ** -22 * (1.0 + np.abs(z) / T))
         + 2.0 ** -8 * np.abs(dz) + (e_g / T)[:, None] * np.abs(onehot - p))
    E[g == 0.0] = 0.0
    return dz, E


def _coef_error(logp, ratio, clipped, A_row, ref, w, beta):
    """e_g: bound on |g_chunk - g| from the forward's logp bar (module doc)."""
    e_logp = 1e-5 * np.abs(logp) + 1e-6
    kl = beta * np.exp(ref - logp) if ref is not None and beta != 0.0 else 0.0
    return (np.where(clipped, 0.0, ratio * np.abs(A_row)) + kl) * np.abs(w) * e_logp


def _assert_bound(got, want, bound, name):
    err = np.abs(np.asarray(got, np.float64) - want)
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:4]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} elements over the bound; "
                             f"err {err.ravel()[i].tolist()} bound {bound.ravel()[i].tolist()}")
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def _check_fused_elementwise(case, h, W, old, ref, gh, gW, chunks):
    """Every element of grad_hidden and grad_weight against the oracle within
    the bound of the module doc; returns the oracle's g."""
    T = case.temperature
    z = h @ W.T
    ref64 = ref.astype(np.float64)
    fwd = oracle.grpo_forward(z, case.ids, old.astype(np.float64), ref64, case.adv, case.mask,
                              case.B, case.L, T, case.beta, case.eps_low, case.eps_high)
    g = oracle.grpo_dlogp(fwd, ref64, case.adv, case.mask, case.dloss, case.B, case.L, case.beta)
    A_row = np.repeat(case.adv.astype(np.float64), case.L)
    e_g = _coef_error(fwd["logp"], fwd["ratio"], fwd["is_clipped"], A_row, ref64,
                      case.dloss.astype(np.float64), case.beta)
    zeta = 2 * case.H * U * (np.abs(h) @ np.abs(W).T)
    onehot = np.zeros_like(z)
    onehot[np.arange(case.N), case.ids] = 1.0
    dz, E = _dz_error(z, zeta, fwd["lse"], g, e_g, onehot, T)
    aW, ah = np.abs(W), np.abs(h)
    gh_o, gW_o = dz @ W, dz.T @ h
    bh = E @ aW + 2 * (case.V + 1) * U * ((np.abs(dz) + E) @ aW)
    bW = E.T @ ah + 2 * (case.N + chunks) * U * ((np.abs(dz) + E).T @ ah)
    rh = _assert_bound(gh, gh_o, bh, "grad_hidden")
    rW = _assert_bound(gW, gW_o, bW, "grad_weight")
    say(f"  largest error / bound: grad_hidden {rh:.3f}, grad_weight {rW:.3f}; Frobenius "
        f"{_frob(gh, gh_o):.2e}, {_frob(gW, gW_o):.2e}")
    # the summary bar holds where |z|/T is moderate (the workloads' T = 0.9);
    # at T = 0.1 or below the bf16 z in the backward's softmax moves p by up to
    # |z| 2^-9 / T, a few percent, and only the element bound applies
    if T >= 0.5:
        assert _frob(gh, gh_o) <= 1e-2 and _frob(gW, gW_o) <= 1e-2
    return g


@pytest.mark.parametrize("chunk,V,T", [(1, 392, 0.9), (2, 392, 0.9), (3, 392, 0.9),
                                       (2, 264, 0.9), (1, 8, 0.9), (2, 392, 0.1),
                                       (3, 264, 0.05)])
def test_fused_small_against_oracle(chunk, V, T):
    """V = 392 leaves 8 columns in the last 128-column half-tile of the
    logits product, V = 264 leaves one half-tile empty, V = 8 has one tile
    with 8 columns: the partial statistics of those must fold exactly the
    columns inside V.  At T = 0.1 and 0.05 every other row samples its most
    likely token, so logp is close to 0 and its 1e-6 floor binds: the
    statistics' sums must be referenced to the exact max, not to its rounded
    product with log2(e)/T."""
    lib = require_gpu()
    case = fill_dloss(synth.fused_case(B=5, L=24, H=128, V=V, dloss="sum"))
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    if T != 0.9:
        case.temperature = T
        ids = case.ids.copy()
        ids[::2] = (h @ W.T)[::2].argmax(axis=1)
        case.ids = ids
    say(f"fused-linear small: B={case.B} L={case.L} H={case.H} V={case.V} chunk={chunk} T={T}")
    logp_true, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
    old, ref = _fused_inputs(case, logp_true)
    loss, gh, gW = _run_fused(lib, case, old, ref, chunk)
    l_o, _, _ = oracle.fused_linear_grpo(h, W, case.ids, old.astype(np.float64),
                                         ref.astype(np.float64), case.adv, case.mask,
                                         case.dloss, case.B, case.L, case.temperature,
                                         case.beta, case.eps_low, case.eps_high, chunk)
    assert abs(loss - l_o) <= 1e-5 * abs(l_o) + 1e-6, (loss, l_o)
    chunks = (case.B + chunk - 1) // chunk
    g = _check_fused_elementwise(case, h, W, old, ref, gh, gW.cpu().numpy(), chunks)
    # rows with dlogp == 0 give exactly zero grad_hidden
    assert (gh[g == 0.0] == 0.0).all()


def test_fused_deterministic():
    lib = require_gpu()
    case = fill_dloss(synth.fused_case(B=4, L=32, H=128, V=512, dloss="mean"))
    say("fused-linear determinism")
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    logp_true, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
    old, ref = _fused_inputs(case, logp_true)
    a = _run_fused(lib, case, old, ref, 2)
    b = _run_fused(lib, case, old, ref, 2)
    assert a[0] == b[0] and np.array_equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_fused_on_a_side_stream_of_the_caller():
    """The chunk runs grad_weight's product on a stream of the library's own
    and joins it back: on a caller stream other than the default one, chunk
    after chunk with no host synchronisation between them, every output is
    bit-identical to the default-stream run."""
    lib = require_gpu()
    case = fill_dloss(synth.fused_case(B=6, L=40, H=128, V=1032, dloss="mean"))
    say("fused-linear on a non-default caller stream")
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    logp_true, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
    old, ref = _fused_inputs(case, logp_true)
    a = _run_fused(lib, case, old, ref, 2)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        b = _run_fused(lib, case, old, ref, 2, stream=side)
    assert a[0] == b[0] and np.array_equal(a[1], b[1]) and torch.equal(a[2], b[2])


@pytest.mark.parametrize("chunk", [4, 3, 2, 1])
def test_fused_full_size(chunk):
    """B=32, L=1024, H=1024, V=151936: loss over all rows against the oracle's
    stored logp; sampled rows of grad_hidden and sampled vocabulary rows of
    grad_weight against the oracle computed one by one."""
    lib = require_gpu()
    case = fill_dloss(synth.fused_case(dloss="mean"))
    say(f"fused-linear full size: B32 L1024 H1024 V151936, chunk {chunk} sequences")
    rows = synth.stored_check_rows("fused")
    logp_true = synth.load_stored_logp("fused", case.hidden[rows])
    lse_true = synth.load_stored_lse("fused")
    old, ref = _fused_inputs(case, logp_true)
    loss, gh, gW = _run_fused(lib, case, old, ref, chunk)
    # oracle per-row quantities from the stored logp
    N = case.N
    A_row = np.repeat(case.adv.astype(np.float64), case.L)
    ratio, pg, clipped = oracle.ppo_clip_terms(logp_true - old, A_row, case.eps_low, case.eps_high)
    d = ref.astype(np.float64) - logp_true
    loss_rows = pg + case.beta * oracle.k3(d)
    l_o = float((case.dloss.astype(np.float64) * loss_rows).sum())
    assert abs(loss - l_o) <= 1e-5 * abs(l_o) + 1e-6, (loss, l_o)
    fwd = dict(logp=logp_true, is_clipped=clipped, ratio=ratio)
    g = oracle.grpo_dlogp(fwd, ref.astype(np.float64), case.adv, case.mask, case.dloss, case.B,
                          case.L, case.beta)
    say(f"  zero rows {(g == 0).sum()} of {N}")
    assert (gh[g == 0.0] == 0.0).all()
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    T = case.temperature
    chunks = (case.B + chunk - 1) // chunk
    e_g = _coef_error(logp_true, ratio, clipped, A_row, ref.astype(np.float64),
                      case.dloss.astype(np.float64), case.beta)
    aW, ah = np.abs(W), np.abs(h)
    rng = np.random.default_rng(5)
    worst = [0.0, 0.0]
    # grad_hidden rows: every element within the bound (module doc)
    rsel = np.concatenate([rng.choice(np.flatnonzero(g != 0.0), 6, replace=False), [0, N - 1]])
    for r in rsel:
        zr = (W @ h[r])[None, :]
        zeta = 2 * case.H * U * (aW @ ah[r])[None, :]
        oh = np.zeros_like(zr)
        oh[0, case.ids[r]] = 1.0
        dz, E = _dz_error(zr, zeta, lse_true[r:r + 1], g[r:r + 1], e_g[r:r + 1], oh, T)
        want = (dz @ W)[0]
        bound = (E @ aW + 2 * (case.V + 1) * U * ((np.abs(dz) + E) @ aW))[0]
        worst[0] = max(worst[0], _assert_bound(gh[r], want, bound, f"grad_hidden row {r}"))
        assert _frob(gh[r], want) <= 1e-2, (r, _frob(gh[r], want))
    # grad_weight rows (vocabulary entries), including sampled-token entries
    vsel = np.concatenate([rng.integers(0, case.V, 4), case.ids[rsel[:4]]])
    gWn = gW[torch.from_numpy(vsel).cuda()].cpu().numpy()
    for k, v in enumerate(vsel):
        zv = (h @ W[v])[:, None]
        zeta = 2 * case.H * U * (ah @ aW[v])[:, None]
        oh = (case.ids == v).astype(np.float64)[:, None]
        dz, E = _dz_error(zv, zeta, lse_true, g, e_g, oh, T)
        want = (dz.T @ h)[0]
        bound = (E.T @ ah + 2 * (N + chunks) * U * ((np.abs(dz) + E).T @ ah))[0]
        worst[1] = max(worst[1], _assert_bound(gWn[k], want, bound, f"grad_weight entry {v}"))
        assert _frob(gWn[k], want) <= 1e-2, (v, _frob(gWn[k], want))
    say(f"  largest error / bound on the sampled rows {worst[0]:.3f}, entries {worst[1]:.3f}")


def _fused_case_with_gaps(B=4, L=40, H=128, V=392):
    """Small case whose weights are 0 on trailing padding and also on rows in
    the middle of sequences (every third valid token) and on the first token
    of sequence 1."""
    case = fill_dloss(synth.fused_case(B=B, L=L, H=H, V=V, dloss="sum"))
    w = case.dloss.copy()
    valid = np.flatnonzero(w != 0.0)
    w[valid[::3]] = 0.0
    w[L] = 0.0
    case.dloss = w
    return case


@pytest.mark.parametrize("chunk", [1, 3])
def test_fused_skips_zero_weight_rows(chunk):
    """Rows with dloss == 0 are compacted away: results match the oracle (which
    computes every row and multiplies by the weight), their grad_hidden rows
    are exactly 0, and a NaN old_logp or an out-of-range id on such a row does
    not reach any output."""
    lib = require_gpu()
    case = _fused_case_with_gaps()
    say(f"fused-linear zero-weight rows skipped: chunk {chunk}, "
        f"{int((case.dloss == 0).sum())} of {case.N} rows have weight 0")
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    logp_true, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
    old, ref = _fused_inputs(case, logp_true)
    l_o, _, _ = oracle.fused_linear_grpo(h, W, case.ids, old.astype(np.float64),
                                         ref.astype(np.float64), case.adv, case.mask,
                                         case.dloss, case.B, case.L, case.temperature,
                                         case.beta, case.eps_low, case.eps_high, chunk)
    dropped = np.flatnonzero(case.dloss == 0.0)
    poisoned_old = old.copy()
    poisoned_old[dropped[0]] = np.nan
    ids_clean = case.ids
    ids_bad = case.ids.copy()
    ids_bad[dropped[1]] = case.V + 7
    case.ids = ids_bad
    loss, gh, gW = _run_fused(lib, case, poisoned_old, ref, chunk)
    case.ids = ids_clean
    assert np.isfinite(loss) and abs(loss - l_o) <= 1e-5 * abs(l_o) + 1e-6, (loss, l_o)
    chunks = (case.B + chunk - 1) // chunk
    _check_fused_elementwise(case, h, W, old, ref, gh, gW.cpu().numpy(), chunks)
    assert (gh[dropped] == 0.0).all()


@pytest.mark.parametrize("bad", [-1, "V"])
def test_fused_invalid_id_on_a_kept_row(bad):
    """An id outside [0, V) on a row that carries weight has no logit to
    gather: like the row forward, its logp is NaN, so the loss is NaN, that
    row's grad_hidden is NaN and (as a sum over rows) every entry of
    grad_weight is NaN; every other row of grad_hidden is unaffected."""
    lib = require_gpu()
    case = fill_dloss(synth.fused_case(B=3, L=24, H=128, V=264, dloss="sum"))
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    logp_true, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
    old, ref = _fused_inputs(case, logp_true)
    kept = np.flatnonzero(case.dloss != 0.0)
    r = int(kept[len(kept) // 2])
    say(f"fused-linear invalid id {bad} on kept row {r}")
    _, gh_ok, _ = _run_fused(lib, case, old, ref, 2)
    ids_bad = case.ids.copy()
    ids_bad[r] = -1 if bad == -1 else case.V
    case.ids = ids_bad
    loss, gh, gW = _run_fused(lib, case, old, ref, 2)
    assert np.isnan(loss)
    assert np.isnan(gh[r]).all()
    others = np.ones(case.N, dtype=bool)
    others[r] = False
    assert np.array_equal(gh[others], gh_ok[others])
    assert torch.isnan(gW).all()


def test_fused_all_rows_zero_weight():
    """A chunk whose weights are all 0 leaves loss_accum and grad_weight as they
    were (bit for bit) and writes grad_hidden = 0."""
    lib = require_gpu()
    case = fill_dloss(synth.fused_case(B=2, L=16, H=64, V=256, dloss="sum"))
    say("fused-linear chunk with every weight 0")
    T = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
             eps_high=case.eps_high)
    rng = np.random.default_rng(3)
    gW0 = rng.standard_normal((case.V, case.H)).astype(np.float32)
    gW = dev(gW0)
    loss = dev(np.array([1.25], dtype=np.float32))
    gh = dev(np.full((case.N, case.H), 7.0, dtype=np.float32))
    ws = torch.empty(lib.fused_linear_grpo_workspace_bytes(case.N, case.V, case.H),
                     dtype=torch.uint8, device="cuda")
    lp = np.zeros(case.N, dtype=np.float32)
    lib.fused_linear_grpo_chunk(_t(case.hidden), _t(case.weight), dev(case.ids), dev(lp),
                                dev(case.adv), dev(case.mask), dev(np.zeros(case.N, np.float32)),
                                case.B, case.L, ref_logp=dev(lp), loss_accum=loss,
                                grad_hidden=gh, grad_weight=gW, workspace=ws, **T)
    torch.cuda.synchronize()
    assert float(loss.item()) == 1.25
    assert (gh.cpu().numpy() == 0.0).all()
    assert np.array_equal(gW.cpu().numpy(), gW0)


@pytest.mark.parametrize("k", range(16))
def test_fused_sweep(k):
    """A seeded sweep of the fused chunk over small shapes: 1-6 sequences of
    1-130 tokens (half of them padding on average, so the kept-row count and
    its rounding up to 64 vary), H of 64-320, V of 8-4104 (ragged last
    tiles), every chunk size from 1 to B, temperatures 0.6-1.3, token-sum
    and token-mean weights.  The loss against the oracle within 1e-5
    relative, every gradient element within the bound of the module doc,
    exact zero grad_hidden rows where dlogp is 0."""
    lib = require_gpu()
    rng = np.random.default_rng(3000 + k)
    B = int(rng.integers(1, 7))
    L = int(rng.choice([1, 7, 24, 65, 130]))
    H = int(rng.choice([64, 128, 192, 320]))
    V = int(rng.choice([8, 136, 264, 392, 520, 1032, 2056, 4104]))
    chunk = int(rng.integers(1, B + 1))
    kind = str(rng.choice(["sum", "mean"]))
    case = fill_dloss(synth.fused_case(seed=k, B=B, L=L, H=H, V=V, dloss=kind))
    case.temperature = float(rng.choice([0.6, 0.9, 1.3]))
    say(f"fused sweep {k}: B={B} L={L} H={H} V={V} chunk={chunk} T={case.temperature} {kind}")
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    logp_true, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
    old, ref = _fused_inputs(case, logp_true)
    loss, gh, gW = _run_fused(lib, case, old, ref, chunk)
    l_o, _, _ = oracle.fused_linear_grpo(h, W, case.ids, old.astype(np.float64),
                                         ref.astype(np.float64), case.adv, case.mask,
                                         case.dloss, case.B, case.L, case.temperature,
                                         case.beta, case.eps_low, case.eps_high, chunk)
    assert abs(loss - l_o) <= 1e-5 * abs(l_o) + 1e-6, (loss, l_o)
    chunks = (case.B + chunk - 1) // chunk
    g = _check_fused_elementwise(case, h, W, old, ref, gh, gW.cpu().numpy(), chunks)
    assert (gh[g == 0.0] == 0.0).all()
