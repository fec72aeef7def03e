"""The entry points called from several host threads at once, each thread on
a stream of its own: the row pass is stateless, and the fused chunk shares
only its per-device side stream (made once, under a mutex) and joins it
back into the caller's stream with events of its own, so every thread's
results must equal those of the same calls made one after another (bit for
bit: the kernels reduce in a fixed order).  ctypes releases the interpreter
lock for the calls, so the library's host code runs concurrently."""
import threading

import numpy as np
import pytest
import torch

import oracle
import synth
from case_weights import fill_dloss
from gpu_common import GrpoInputs, logits_to_dev, require_gpu, say

pytestmark = pytest.mark.gpu

THREADS = 4
CALLS = 12


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _row_job(lib, seed):
    """Inputs of one thread's token-level single pass and two-pass calls."""
    case = fill_dloss(synth.grpo_token_case(seed=seed, with_ref=True, dloss="mean"))
    z64 = oracle.decode_bf16(case.logits)
    logp, _ = oracle.selective_log_softmax(z64[:, :], case.ids, case.temperature)
    inp = GrpoInputs(case, logp)
    return case, logits_to_dev(case.logits, "bf16"), inp.to_dev()


def _row_calls(lib, case, t, d, stream):
    kw = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
              eps_high=case.eps_high)
    with torch.cuda.stream(stream):
        o, dz, zr = lib.grpo_logits_fwd_bwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L,
                                            d["dloss"], ref_logp=d["ref_logp"], mask=d["mask"],
                                            **kw)
        f = lib.grpo_logits_fwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L,
                                ref_logp=d["ref_logp"], mask=d["mask"], **kw)
        dz2, _ = lib.grpo_logits_bwd(t, d["ids"], d["old_logp"], d["adv"], case.B, case.L,
                                     f["logp"], f["lse"], d["dloss"], ref_logp=d["ref_logp"],
                                     mask=d["mask"], **kw)
    return [o["loss"], o["logp"], o["lse"], dz, zr, f["loss"], dz2]


class _FusedJob:
    def __init__(self, seed):
        c = fill_dloss(synth.fused_case(seed=seed, B=2, L=130, H=192, V=4104, dloss="sum"))
        h, W = oracle.decode_bf16(c.hidden), oracle.decode_bf16(c.weight)
        lp, _ = oracle.selective_log_softmax(h @ W.T, c.ids, c.temperature)
        dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.c = c
        self.h, self.W = _bf16(c.hidden), _bf16(c.weight)
        self.ids, self.adv, self.dl = dv(c.ids), dv(c.adv), dv(c.dloss)
        self.old = dv(synth.add_noise_f32(lp, c.old_noise))
        self.ref = dv(synth.add_noise_f32(lp, c.ref_noise))

    def call(self, lib, stream):
        c = self.c
        with torch.cuda.stream(stream):
            loss = torch.zeros(1, device="cuda")
            gW = torch.zeros((c.V, c.H), device="cuda")
            _, gh, gW = lib.fused_linear_grpo_chunk(
                self.h, self.W, self.ids, self.old, self.adv, None, self.dl, c.B, c.L,
                ref_logp=self.ref, temperature=c.temperature, beta=c.beta, eps_low=c.eps_low,
                eps_high=c.eps_high, loss_accum=loss, grad_weight=gW)
        return [loss, gh, gW]


def _same(got, want, what):
    for k, (a, b) in enumerate(zip(got, want)):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
            f"{what}: output {k} differs from the sequential call"


def _run_threads(work):
    """Run work(i) for i in range(THREADS) on that many host threads; re-raise
    the first failure."""
    errors = []

    def body(i):
        try:
            work(i)
        except BaseException as e:  # noqa: BLE001 - reported to the main thread
            errors.append(e)

    threads = [threading.Thread(target=body, args=(i,)) for i in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    if errors:
        raise errors[0]


def test_row_entry_points_from_several_threads():
    lib = require_gpu()
    say(f"row entry points from {THREADS} host threads x {CALLS} calls, one stream each "
        f"(B4 L512 V32000 bf16, seeds 0..{THREADS - 1})")
    jobs = [_row_job(lib, seed) for seed in range(THREADS)]
    default = torch.cuda.current_stream()
    want = [[x.clone() for x in _row_calls(lib, *job, default)] for job in jobs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(THREADS)]
    got = [[None] * CALLS for _ in range(THREADS)]

    def work(i):
        for k in range(CALLS):
            got[i][k] = _row_calls(lib, *jobs[i], streams[i])

    _run_threads(work)
    torch.cuda.synchronize()
    for i in range(THREADS):
        for k in range(CALLS):
            _same(got[i][k], want[i], f"thread {i} call {k}")
    say(f"  {THREADS * CALLS} concurrent calls bit-identical to the sequential ones")


def test_fused_chunk_from_several_threads():
    lib = require_gpu()
    say(f"fused chunk from {THREADS} host threads x {CALLS // 2} calls, one stream each "
        f"(B2 L130 H192 V4104, seeds 0..{THREADS - 1}); they share the side stream")
    jobs = [_FusedJob(seed) for seed in range(THREADS)]
    default = torch.cuda.current_stream()
    want = [[x.clone() for x in job.call(lib, default)] for job in jobs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(THREADS)]
    got = [[None] * (CALLS // 2) for _ in range(THREADS)]

    def work(i):
        for k in range(CALLS // 2):
            got[i][k] = jobs[i].call(lib, streams[i])

    _run_threads(work)
    torch.cuda.synchronize()
    for i in range(THREADS):
        for k in range(CALLS // 2):
            _same(got[i][k], want[i], f"thread {i} call {k}")
    say(f"  {THREADS * (CALLS // 2)} concurrent fused calls bit-identical to the sequential ones")
