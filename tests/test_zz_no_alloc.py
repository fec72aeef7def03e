"""The fused-linear chunk's entry point that allocates nothing
(fused_linear_grpo_chunk_noalloc, the workspace in a static device array of
the library's own) against fused_linear_grpo_chunk with a caller workspace:
both run the same kernels in the same order, so every output must be
bit-identical -- on two calls in a row on one stream, the second with a
smaller input (so the array still holds the first call's data), and again
after the workspace entry point has run.  A chunk that needs more than the
array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import synth
from case_weights import fill_dloss
from gpu_common import dev, require_gpu, say

pytestmark = pytest.mark.gpu


def _t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class _Chunk:
    """Device inputs of one chunk (all the case's sequences) and fresh outputs."""

    def __init__(self, case, old, ref):
        self.case = case
        self.h, self.W = _t(case.hidden), _t(case.weight)
        self.ids, self.old, self.ref = dev(case.ids), dev(old), dev(ref)
        self.adv, self.mask, self.dl = dev(case.adv), dev(case.mask), dev(case.dloss)
        self.kw = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
                       eps_high=case.eps_high)

    def outputs(self):
        c = self.case
        gW0 = torch.from_numpy(np.random.default_rng(c.V).standard_normal((c.V, c.H))
                               .astype(np.float32)).cuda()   # grad_weight accumulates into it
        return (torch.full((1,), 0.5, device="cuda"),
                torch.full((c.N, c.H), 3.0, device="cuda"), gW0)

    def run(self, lib, noalloc):
        c = self.case
        loss, gh, gW = self.outputs()
        args = (self.h, self.W, self.ids, self.old, self.adv, self.mask, self.dl, c.B, c.L)
        kw = dict(ref_logp=self.ref, loss_accum=loss, grad_hidden=gh, grad_weight=gW, **self.kw)
        if noalloc:
            lib.fused_linear_grpo_chunk_noalloc(*args, **kw)
        else:
            lib.fused_linear_grpo_chunk(*args, **kw)
        return loss, gh, gW


def _chunk(case):
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    lp, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
    old = synth.add_noise_f32(lp, case.old_noise)
    ref = synth.add_noise_f32(lp, case.ref_noise)
    return _Chunk(case, old, ref)


def _same(a, b, what):
    for x, y, n in zip(a, b, ("loss_accum", "grad_hidden", "grad_weight")):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"{what}: {n} differs"


def test_noalloc_matches_workspace_entry_point():
    lib = require_gpu()
    # the first call: one 1024-token sequence of the Qwen3-0.6B-sized head
    # (V = 151936, H = 1024: about 363 of the array's 384 MiB); the second a
    # smaller chunk (3 sequences of 24 tokens, V = 392, H = 128)
    big = fill_dloss(synth.fused_case(B=1, L=1024, dloss="mean"))
    small = fill_dloss(synth.fused_case(B=3, L=24, H=128, V=392, dloss="sum"))
    need = lib.fused_linear_grpo_workspace_bytes(big.N, big.V, big.H)
    say(f"no-alloc fused chunk: B1 L1024 H1024 V151936 ({need / 2**20:.0f} MiB of "
        f"{lib.NOALLOC_SCRATCH_BYTES / 2**20:.0f}) then B3 L24 H128 V392, in a row")
    assert need <= lib.NOALLOC_SCRATCH_BYTES
    cb, cs = _chunk(big), _chunk(small)
    # two calls in a row on one stream, no host synchronisation between them
    nb = cb.run(lib, True)
    ns = cs.run(lib, True)
    torch.cuda.synchronize()
    wb = cb.run(lib, False)
    ws = cs.run(lib, False)
    torch.cuda.synchronize()
    _same(nb, wb, "1024-token chunk")
    _same(ns, ws, "small chunk after it")
    assert torch.isfinite(nb[1]).all() and float(nb[0].item()) != 0.5
    # and once more after the workspace entry point, on the stale array
    ns2 = cs.run(lib, True)
    torch.cuda.synchronize()
    _same(ns2, ws, "small chunk again")


def test_noalloc_refuses_a_chunk_beyond_its_scratch():
    lib = require_gpu()
    B, L, H, V = 2, 1024, 1024, 151936
    need = lib.fused_linear_grpo_workspace_bytes(B * L, V, H)
    say(f"no-alloc fused chunk refuses {need / 2**20:.0f} MiB > 384 MiB")
    assert need > lib.NOALLOC_SCRATCH_BYTES
    h = torch.zeros((B * L, H), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((V, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(B * L, dtype=torch.int64, device="cuda")
    f = torch.zeros(B * L, device="cuda")
    adv = torch.zeros(B, device="cuda")
    loss = torch.full((1,), 2.5, device="cuda")
    gh = torch.full((B * L, H), 7.0, device="cuda")
    gW = torch.full((V, H), 1.5, device="cuda")
    with pytest.raises(lib.GrpoError) as e:
        lib.fused_linear_grpo_chunk_noalloc(h, W, ids, f, adv, None, f, B, L, loss_accum=loss,
                                            grad_hidden=gh, grad_weight=gW, temperature=0.9)
    assert e.value.status == 9
    torch.cuda.synchronize()
    assert float(loss.item()) == 2.5 and bool((gh == 7.0).all()) and bool((gW == 1.5).all())
