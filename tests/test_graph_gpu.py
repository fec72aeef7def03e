"""The entry points recorded into a HIP graph (torch's CUDA graph API on ROCm)
and replayed: the two-pass forward and backward, the single pass, the
entropy and selective log-softmax pairs, the steps either side (group
advantages, loss weights), and the fused-linear chunk's entry point that
allocates nothing -- the one meant for callers under graph capture.

Each entry point enqueues kernels only (no allocation, no memset, no host
synchronisation), and none of them uses atomics on valid inputs or a
reduction order that varies between launches, so every replay must
reproduce the eager call's outputs bit for bit.  Between replays the outputs
are overwritten with junk, and other eager calls run on other buffers (for
the fused chunk: a smaller chunk through the same static scratch), with host
synchronisations in between."""
import numpy as np
import pytest
import torch

import oracle
import synth
from case_weights import fill_dloss
from gpu_common import GrpoInputs, logits_to_dev, require_gpu, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _same(got, want, what):
    assert got.shape == want.shape and got.dtype == want.dtype, what
    a = got.contiguous().view(torch.uint8)
    b = want.contiguous().view(torch.uint8)
    assert torch.equal(a, b), f"{what}: replay differs from the eager call"


def _junk(tensors):
    for t in tensors:
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(7)


class _RowRun:
    """Every row entry point on one case, into outputs allocated once."""

    def __init__(self, lib, case: synth.GrpoCase, inp: GrpoInputs, dtype: str):
        self.lib, self.c = lib, case
        self.t = logits_to_dev(case.logits, dtype)
        self.d = inp.to_dev()
        self.rewards = torch.linspace(-1.0, 2.0, case.B * 4, device="cuda")
        N, B = case.N, case.B
        f32, u8 = torch.float32, torch.uint8
        e = lambda n, dt=f32: torch.empty(n, dtype=dt, device="cuda")
        z = lambda: torch.empty_like(self.t)
        self.fwd = dict(loss=e(N), logp=e(N), lse=e(N), entropy=e(N), kl=e(N),
                        is_clipped=e(N, u8), gathered=e(N))
        if case.level == "sequence":
            self.fwd["seq_ratio"] = e(B)
        self.err, self.dz, self.zr = e(1, torch.int32), z(), e(N, u8)
        self.single = None
        if case.level == "token":
            self.single = dict(loss=e(N), logp=e(N), lse=e(N), entropy=e(N), kl=e(N),
                               is_clipped=e(N, u8))
            self.err1, self.dz1, self.zr1 = e(1, torch.int32), z(), e(N, u8)
        self.ent, self.slp, self.slse = e(N), e(N), e(N)
        self.sdz, self.edz = z(), z()
        self.adv_g, self.w = e(B * 4), e(N)

    def outputs(self):
        o = dict(self.fwd)
        o.update(err=self.err, dz=self.dz, zr=self.zr, ent=self.ent, slp=self.slp,
                 slse=self.slse, sdz=self.sdz, edz=self.edz, adv_g=self.adv_g, w=self.w)
        if self.single is not None:
            o.update({f"single_{k}": v for k, v in self.single.items()})
            o.update(err1=self.err1, dz1=self.dz1, zr1=self.zr1)
        return o

    def launch(self, temperature=None):
        lib, c, d, t = self.lib, self.c, self.d, self.t
        T = c.temperature if temperature is None else temperature
        kw = dict(temperature=T, beta=c.beta, eps_low=c.eps_low, eps_high=c.eps_high)
        self.err.zero_()
        lib.grpo_logits_fwd(t, d["ids"], d["old_logp"], d["adv"], c.B, c.L,
                            ref_logp=d["ref_logp"], mask=d["mask"], level=c.level,
                            gathered=True, err_count=self.err, out=self.fwd, **kw)
        lib.grpo_logits_bwd(t, d["ids"], d["old_logp"], d["adv"], c.B, c.L, self.fwd["logp"],
                            self.fwd["lse"], d["dloss"], ref_logp=d["ref_logp"], mask=d["mask"],
                            seq_ratio=self.fwd.get("seq_ratio"), level=c.level, dlogits=self.dz,
                            zero_row=self.zr, **kw)
        if self.single is not None:
            self.err1.zero_()
            lib.grpo_logits_fwd_bwd(t, d["ids"], d["old_logp"], d["adv"], c.B, c.L, d["dloss"],
                                    ref_logp=d["ref_logp"], mask=d["mask"], dlogits=self.dz1,
                                    zero_row=self.zr1, err_count=self.err1, out=self.single, **kw)
        lib.entropy_from_logits(t, T, out=self.ent)
        lib.selective_log_softmax(t, d["ids"], T, out=self.slp, lse=self.slse)
        lib.selective_log_softmax_bwd(t, d["ids"], self.slse, d["dloss"], T, dlogits=self.sdz)
        lib.entropy_from_logits_bwd(t, self.slse, self.ent, d["dloss"], T, dlogits=self.edz)
        lib.grpo_group_advantages(self.rewards, 4, adv=self.adv_g)
        lib.grpo_loss_weights(d["mask"], c.B, c.L, "sequence", dloss=self.w)


def _replay_rows(lib, case, inp, dtype, what):
    eager = _RowRun(lib, case, inp, dtype)
    eager.launch()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in eager.outputs().items()}
    assert int(want["err"].item()) == 0
    assert torch.isfinite(want["loss"]).all() and torch.isfinite(want["dz"].float()).all()

    cap = _RowRun(lib, case, inp, dtype)
    other = _RowRun(lib, case, inp, dtype)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap.launch()
    torch.cuda.synchronize()
    for k in range(REPLAYS):
        _junk(cap.outputs().values())
        other.launch(temperature=case.temperature * (1.5 + k))   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in cap.outputs().items():
            _same(t, want[name], f"{what}, replay {k + 1}: {name}")
    say(f"  {what}: {REPLAYS} replays bit-identical to the eager calls "
        f"({len(want)} outputs each)")
    del g


def test_row_entry_points_replay_from_a_graph():
    lib = require_gpu()
    case = fill_dloss(synth.grpo_token_case(with_ref=True, dloss="mean"))
    logp = synth.load_stored_logp("token", case.logits[synth.stored_check_rows("token")])
    say("graph capture: row entry points on B4 L512 V32000 bf16 (token level, reference model)")
    _replay_rows(lib, case, GrpoInputs(case, logp), "bf16", "token level B4 L512 V32000 bf16")


def test_sequence_level_replays_from_a_graph():
    lib = require_gpu()
    case = fill_dloss(synth.tiny_case("s"))
    z64 = case.logits.astype(np.float64)
    logp, _ = oracle.selective_log_softmax(z64, case.ids, case.temperature)
    say(f"graph capture: sequence level B{case.B} L{case.L} V{case.V} fp32")
    _replay_rows(lib, case, GrpoInputs(case, logp), "f32",
                 f"sequence level B{case.B} L{case.L} V{case.V} fp32")


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class _FusedRun:
    """One chunk's device inputs and outputs for the entry point that
    allocates nothing; loss_accum and grad_weight accumulate, so every launch
    first sets them (fill kernels, no memset) to fixed values."""

    def __init__(self, case: synth.FusedCase):
        self.c = case
        h, W = oracle.decode_bf16(case.hidden), oracle.decode_bf16(case.weight)
        lp, _ = oracle.selective_log_softmax(h @ W.T, case.ids, case.temperature)
        dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.h, self.W = _bf16(case.hidden), _bf16(case.weight)
        self.ids, self.adv, self.mask, self.dl = dv(case.ids), dv(case.adv), dv(case.mask), dv(case.dloss)
        self.old = dv(synth.add_noise_f32(lp, case.old_noise))
        self.ref = dv(synth.add_noise_f32(lp, case.ref_noise))
        self.loss = torch.empty(1, device="cuda")
        self.gh = torch.empty((case.N, case.H), device="cuda")
        self.gW = torch.empty((case.V, case.H), device="cuda")

    def outputs(self):
        return dict(loss_accum=self.loss, grad_hidden=self.gh, grad_weight=self.gW)

    def launch(self, lib):
        c = self.c
        self.loss.fill_(0.5)
        self.gW.fill_(0.25)
        lib.fused_linear_grpo_chunk_noalloc(
            self.h, self.W, self.ids, self.old, self.adv, self.mask, self.dl, c.B, c.L,
            ref_logp=self.ref, temperature=c.temperature, beta=c.beta, eps_low=c.eps_low,
            eps_high=c.eps_high, loss_accum=self.loss, grad_hidden=self.gh, grad_weight=self.gW)


def test_fused_noalloc_replays_from_a_graph():
    lib = require_gpu()
    main = fill_dloss(synth.fused_case(seed=3, B=2, L=130, H=192, V=4104, dloss="sum"))
    small = fill_dloss(synth.fused_case(seed=4, B=3, L=24, H=128, V=392, dloss="mean"))
    say("graph capture: fused chunk without allocation, B2 L130 H192 V4104 "
        "(eager B3 L24 H128 V392 through the same scratch between replays)")
    eager = _FusedRun(main)
    eager.launch(lib)          # the first call also looks up the scratch's device address
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in eager.outputs().items()}
    assert torch.isfinite(want["grad_hidden"]).all() and float(want["loss_accum"].item()) != 0.5

    cap, other = _FusedRun(main), _FusedRun(small)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap.launch(lib)
    torch.cuda.synchronize()
    for k in range(REPLAYS):
        _junk(cap.outputs().values())
        other.launch(lib)      # overwrites the static scratch the graph's kernels use
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in cap.outputs().items():
            _same(t, want[name], f"fused chunk, replay {k + 1}: {name}")
    say(f"  fused chunk: {REPLAYS} replays bit-identical to the eager call")
    del g
