"""GPU parity of the bf16 MFMA GEMM and of the chunked fused-linear GRPO loss.

GEMM: against float64 products of the same bf16 values; the bound is the
fp32 accumulation error, |err| <= 2 K 2^-24 sum_k |a_mk b_kn| (+ the same for
the accumulated C).
Fused linear: loss within 1e-5 relative (fp32 logits into the row pass);
grad_hidden and grad_weight within 1e-2 relative Frobenius error per tensor
(dz is rounded to bf16, 2^-9 relative per element, before the two products);
rows of grad_hidden whose dlogp is 0 are exactly 0.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import dev, require_gpu, say

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    bits = synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))
    return bits, oracle.decode_bf16(bits)


def _t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("a_layout,b_layout", [(0, 0), (0, 1), (1, 1), (1, 0)])
@pytest.mark.parametrize("M,N,K", [(128, 128, 32), (200, 264, 96), (520, 392, 1064), (8, 16, 8),
                                   (4000, 7880, 136), (2056, 14344, 72), (4096, 8192, 200)])
def test_gemm_layouts(a_layout, b_layout, M, N, K):
    """The first four shapes take the 128 x 128 block tile; (4000, 7880, 136)
    has fewer than 512 tiles of 256 x 256 but at least 512 of 256 x 128, so a
    transposed operand takes the 256 x 128 tile (K-contiguous ones the
    128 x 128); the last two (>= 512 tiles of 256 x 256, ragged in M, N and K)
    take the pipelined 256 x 256 x 64 tile in every layout."""
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


def _fused_inputs(case, logp_true):
    old = synth.add_noise_f32(logp_true, case.old_noise)
    ref = synth.add_noise_f32(logp_true, case.ref_noise)
    return old, ref


def _run_fused(lib, case, old, ref, chunk):
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
                                    grad_hidden=gh[rs], grad_weight=gW, workspace=ws, **T)
    torch.cuda.synchronize()
    return float(loss.item()), gh.cpu().numpy(), gW


def _frob(got, want):
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


@pytest.mark.parametrize("chunk", [1, 2, 3])
def test_fused_small_against_oracle(chunk):
    lib = require_gpu()
    case = synth.fused_case(B=5, L=24, H=128, V=392, dloss="sum")
    say(f"fused-linear small: B={case.B} L={case.L} H={case.H} V={case.V} chunk={chunk}")
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight) * 1.0
    logp_true, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
    old, ref = _fused_inputs(case, logp_true)
    loss, gh, gW = _run_fused(lib, case, old, ref, chunk)
    l_o, gh_o, gW_o = oracle.fused_linear_grpo(h, W, case.ids, old.astype(np.float64),
                                               ref.astype(np.float64), case.adv, case.mask,
                                               case.dloss, case.B, case.L, case.temperature,
                                               case.beta, case.eps_low, case.eps_high, chunk)
    assert abs(loss - l_o) <= 1e-5 * abs(l_o) + 1e-6, (loss, l_o)
    assert _frob(gh, gh_o) <= 1e-2, _frob(gh, gh_o)
    assert _frob(gW.cpu().numpy(), gW_o) <= 1e-2
    # rows with dlogp == 0 give exactly zero grad_hidden
    z = h @ W.T
    fwd = oracle.grpo_forward(z, case.ids, old.astype(np.float64), ref.astype(np.float64),
                              case.adv, case.mask, case.B, case.L, case.temperature, case.beta,
                              case.eps_low, case.eps_high)
    g = oracle.grpo_dlogp(fwd, ref.astype(np.float64), case.adv, case.mask, case.dloss, case.B,
                          case.L, case.beta)
    assert (gh[g == 0.0] == 0.0).all()


def test_fused_deterministic():
    lib = require_gpu()
    case = synth.fused_case(B=4, L=32, H=128, V=512, dloss="mean")
    say("fused-linear determinism")
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    logp_true, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
    old, ref = _fused_inputs(case, logp_true)
    a = _run_fused(lib, case, old, ref, 2)
    b = _run_fused(lib, case, old, ref, 2)
    assert a[0] == b[0] and np.array_equal(a[1], b[1]) and torch.equal(a[2], b[2])


@pytest.mark.parametrize("chunk", [4, 3, 2, 1])
def test_fused_full_size(chunk):
    """B=32, L=1024, H=1024, V=151936: loss over all rows against the oracle's
    stored logp; sampled rows of grad_hidden and sampled vocabulary rows of
    grad_weight against the oracle computed one by one."""
    lib = require_gpu()
    case = synth.fused_case(dloss="mean")
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
    rng = np.random.default_rng(5)
    # grad_hidden rows
    rsel = np.concatenate([rng.choice(np.flatnonzero(g != 0.0), 6, replace=False), [0, N - 1]])
    for r in rsel:
        zr = W @ h[r]
        p = np.exp(zr / T - lse_true[r])
        dz = -(g[r] / T) * p
        dz[case.ids[r]] += g[r] / T
        want = dz @ W
        assert _frob(gh[r], want) <= 1e-2, (r, _frob(gh[r], want))
    # grad_weight rows (vocabulary entries), including sampled-token entries
    vsel = np.concatenate([rng.integers(0, case.V, 4), case.ids[rsel[:4]]])
    gWn = gW[torch.from_numpy(vsel).cuda()].cpu().numpy()
    for k, v in enumerate(vsel):
        zv = h @ W[v]
        p = np.exp(zv / T - lse_true)
        dzv = -(g / T) * p
        hit = case.ids == v
        dzv[hit] += g[hit] / T
        want = dzv @ h
        assert _frob(gWn[k], want) <= 1e-2, (v, _frob(gWn[k], want))
