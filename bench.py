"""Benchmark of the GRPO logits row pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--sets S] [--chunk C] [--no-cpu-baseline] [--copy-probe]

Default workload ``grpo-token`` (the headline): a step is one forward +
backward of the token-level GRPO loss over the logits of B=4 sequences x
L=512 tokens x V=32000 vocabulary entries (bf16, T=0.9, beta=0.04, eps
0.2/0.28, half the advantages exactly 0, no reference model so the KL term
vanishes, token-mean upstream gradient), run as the single pass
grpo_logits_fwd_bwd: loss, logp, lse, entropy, kl and is_clipped per token
and dlogits (all-zero rows where dlogp is 0) from one read of the logits.
The two-pass step (grpo_logits_fwd then grpo_logits_bwd) is timed too and
reported under "two_pass".  S buffer sets (about 1 GB
in total by default) rotate from step to step so a step does not find the
previous step's logits in the 256 MB last-level cache.

Other workloads (each prints its own line; not the headline):
  grpo-seq      sequence-level fwd+bwd, B=8 L=1024 V=151936 bf16, beta=0
  rows          entropy_from_logits + selective_log_softmax fwd + bwd,
                65536 x 32000 bf16 (contiguous; --strided: rows of a 2V buffer)
  fused-linear  chunked fused-linear loss over h [32768, 1024] and
                W [151936, 1024] bf16, --chunk sequences per call (value:
                rows/s; roofline on the dominant kernel, the logits product
                with its row statistics, timed alone on the first chunk's
                kept rows; zero-weight rows are skipped)
  entropy-bwd   entropy_from_logits_bwd over the rows workload's logits,
                plus the latency of grpo_group_advantages / grpo_loss_weights
  tiny          the B=2 L=16 V=1024 fp32 GRPO step (value: microseconds per
                step, lower is better; launch-latency bound)

Inputs are synthetic, generated on the host and already resident in device
memory when the timed region starts.  ``value`` is GB/s of algorithmic HBM
bytes (rows/s for fused-linear) over the wall time of the timed steps.  ``roofline`` is for the step's dominant kernel, its
duration timed with events on the launch stream over back-to-back launches; ``traffic`` is the HBM bytes
per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters stored in
profiles/counters.json, used only while the kernels' source digest matches.
``cpu_baseline`` times the float64 oracle on a bounded sample of the same
workload on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="grpo-token",
                    choices=["grpo-token", "grpo-seq", "rows", "fused-linear", "entropy-bwd",
                             "tiny"])
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--chunk", type=int, default=4)
    ap.add_argument("--strided", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of 256 MiB (counter calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def digest_part(workload: str) -> str:
    """Which sources a workload's kernels come from: the fused-linear path
    runs the GEMMs and the row kernels, every other workload the row kernels."""
    return "all" if workload == "fused-linear" else "rows"


def stored_counters(workload: str):
    """Per-kernel entries of the stored counter runs for a workload, if the
    kernels have not changed since (source digest of the workload's sources);
    else {}."""
    from rl_fine_tuning_row_amd.build import source_digest
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    part = digest_part(workload)
    if data.get("source_digests", {}).get(part) != source_digest(part):
        return {}
    pre = workload + ":"
    return {k[len(pre):]: v for k, v in data.get("kernels", {}).items() if k.startswith(pre)}


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the stored counter runs (None if stale)."""
    e = stored_counters(workload).get(kernel)
    if e is None or "fetch_bytes" not in e:
        return None
    return e["fetch_bytes"] + e["write_bytes"]


def timed(step_fns, steps, torch):
    """Wall time (ms) per step of `steps` steps rotating over step_fns."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step_fns[i % len(step_fns)]()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def kernel_times(launch_lists, steps, torch):
    """Average duration (ms) of each launch position of a step: that launch
    alone, `steps` times back to back (rotating over the buffer sets), between
    two events on the launch stream.  Inputs of every position were produced
    by the warm-up steps and no launch changes another's inputs."""
    out = []
    for k in range(len(launch_lists[0])):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            launch_lists[i % len(launch_lists)][k]()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return out


def copy_probe(torch):
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def base_line(args, metric, value, unit, ms, config, dtype="bf16"):
    return {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "config": config}


# per-row scalar bytes of the GRPO kernels
FWD_ROW_BYTES = 8 + 4 + 5 * 4 + 1      # ids, old_logp in; loss, logp, lse, entropy, kl, is_clipped out
BWD_ROW_BYTES = 8 + 4 + 4 + 4 + 4 + 1  # ids, old_logp, logp, lse, dloss in; zero_row out
ONE_ROW_BYTES = 8 + 4 + 4 + 5 * 4 + 1 + 1  # ids, old_logp, dloss in; 5 fp32, is_clipped, zero_row out


# ---------------------------------------------------------------------------
# GRPO token / sequence level
# ---------------------------------------------------------------------------
def run_grpo(args, torch, grl, synth, level):
    """Token level: the step is the single-pass grpo_logits_fwd_bwd (dloss of
    a token-mean loss is known before the forward); the two-pass
    grpo_logits_fwd + grpo_logits_bwd step is timed as well and reported under
    "two_pass".  Sequence level (needs the per-sequence ratio before any
    gradient): the two-pass step."""
    if level == "token":
        case = synth.grpo_token_case(with_ref=False, dloss="mean")
        name = "token"
    else:
        case = synth.grpo_sequence_case(dloss="mean")
        name = "sequence"
    logp_true = synth.load_stored_logp(name, case.logits[synth.stored_check_rows(name)])
    old = synth.add_noise_f32(logp_true, case.old_noise)
    B, L, V, N = case.B, case.L, case.V, case.N
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    z0 = torch.from_numpy(case.logits.view(np.int16)).view(torch.bfloat16).cuda()
    ids, old_t, adv, mask, dloss = (dev(case.ids), dev(old), dev(case.adv), dev(case.mask),
                                    dev(case.dloss))
    nsets = args.sets if level == "token" else 2
    kw = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
              eps_high=case.eps_high)
    sets = []
    for k in range(nsets):
        z = z0.clone() if k else z0
        out = {n: torch.empty(N, dtype=torch.float32, device="cuda")
               for n in ("loss", "logp", "lse", "entropy", "kl")}
        out["is_clipped"] = torch.empty(N, dtype=torch.uint8, device="cuda")
        dz = torch.empty((N, V), dtype=torch.bfloat16, device="cuda")
        zr = torch.empty(N, dtype=torch.uint8, device="cuda")
        # arguments marshalled once; a step is one (single pass) or two C calls
        fwd, out = grl.grpo_logits_fwd(z, ids, old_t, adv, B, L, mask=mask, out=out,
                                       prepare=True, level=level, **kw)
        bwd, _, _ = grl.grpo_logits_bwd(z, ids, old_t, adv, B, L, out["logp"], out["lse"],
                                        dloss, mask=mask, seq_ratio=out.get("seq_ratio"),
                                        dlogits=dz, zero_row=zr, prepare=True, level=level, **kw)
        # the backward with the all-zero path switched off, for the skip A/B
        dense, _, _ = grl.grpo_logits_bwd(z, ids, old_t, adv, B, L, out["logp"], out["lse"],
                                          dloss, mask=mask, seq_ratio=out.get("seq_ratio"),
                                          dlogits=dz, zero_row=zr, prepare=True, level=level,
                                          force_dense=True, **kw)
        one = None
        if level == "token":
            one, _, _, _ = grl.grpo_logits_fwd_bwd(z, ids, old_t, adv, B, L, dloss, mask=mask,
                                                   out=out, dlogits=dz, zero_row=zr,
                                                   prepare=True, **kw)
        sets.append(dict(fwd=fwd, bwd=bwd, dense=dense, one=one, zr=zr))
    two_steps = [(lambda s=s: (s["fwd"](), s["bwd"]())) for s in sets]
    for i in range(args.warmup):
        two_steps[i % len(two_steps)]()
        if level == "token":
            sets[i % len(sets)]["one"]()
    torch.cuda.synchronize()
    n_zero = int(sets[0]["zr"].sum().item())
    n_nz = N - n_zero
    fwd_bytes = N * V * 2 + N * FWD_ROW_BYTES
    bwd_bytes = N * V * 2 + n_nz * V * 2 + N * BWD_ROW_BYTES
    two_bytes = fwd_bytes + bwd_bytes
    ms_two = timed(two_steps, args.steps, torch)
    fwd_ms, bwd_ms = kernel_times([[s["fwd"], s["bwd"]] for s in sets], args.steps, torch)
    two_pass = {
        "ms_per_step": round(ms_two, 5), "step_bytes": two_bytes,
        "GB/s": round(two_bytes / (ms_two * 1e-3) / 1e9, 1),
        "rows_per_s": round(N / (ms_two * 1e-3), 1),
        "kernels": {"grpo_fwd": {"ms": round(fwd_ms, 5), "bytes": fwd_bytes,
                                 "GB/s": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1)},
                    "grpo_bwd": {"ms": round(bwd_ms, 5), "bytes": bwd_bytes,
                                 "GB/s": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9, 1)}}}
    if level == "token":
        # single pass: logits read once, dlogits written once
        one_bytes = 2 * N * V * 2 + N * ONE_ROW_BYTES
        ms = timed([s["one"] for s in sets], args.steps, torch)
        (one_ms,) = kernel_times([[s["one"]] for s in sets], args.steps, torch)
        # warm: one buffer set over and over, its 131 MB of logits left in the
        # 256 MB last-level cache by the step before (reported, not the value)
        (warm_ms,) = kernel_times([[sets[0]["one"]]], args.steps, torch)
        step_bytes = one_bytes
        kern = {"grpo_fwd_bwd": (one_ms, one_bytes)}
    else:
        ms = ms_two
        step_bytes = two_bytes
        kern = {"grpo_fwd": (fwd_ms, fwd_bytes), "grpo_bwd": (bwd_ms, bwd_bytes)}
    gbs = step_bytes / (ms * 1e-3) / 1e9
    dom = max(kern, key=lambda k: kern[k][0])
    dom_gbs = kern[dom][1] / (kern[dom][0] * 1e-3) / 1e9
    wl = "grpo-token" if level == "token" else "grpo-seq"
    if level == "token":
        metric = "GRPO logits fwd+bwd GB/s & % HBM peak at B4 L512 V32000 bf16; rows/s"
        desc = ("token-level GRPO logits fwd+bwd in one pass (grpo_logits_fwd_bwd), B=4 L=512 "
                "V=32000 bf16 (T=0.9, beta=0.04, eps 0.2/0.28, 2 of 4 advantages 0, "
                "ref = policy, token-mean dloss, lengths U{256..512})")
    else:
        metric = "GRPO sequence-level logits fwd+bwd GB/s at B8 L1024 V151936 bf16; rows/s"
        desc = ("sequence-level GRPO logits fwd+bwd, B=8 L=1024 V=151936 bf16 (T=1, beta=0, "
                "eps 0.2/0.28, 2 of 8 advantages 0, one old-logp offset per sequence)")
    res = base_line(args, metric, gbs, "GB/s", ms,
                    {"workload": desc, "rows": N, "V": V, "zero_rows": n_zero,
                     "nonzero_rows": n_nz, "buffer_sets": nsets, "accumulate": "fp32"})
    res.update({
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "rows_per_s": round(N / (ms * 1e-3), 1),
        "step_bytes": step_bytes,
        "kernels": {k: {"ms": round(v[0], 5), "bytes": v[1],
                        "GB/s": round(v[1] / (v[0] * 1e-3) / 1e9, 1)} for k, v in kern.items()},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(dom, wl)},
    })
    if level == "token":
        res["two_pass"] = two_pass
        res["warm_single_set"] = {
            "note": "one buffer set repeated: the logits stay in the last-level cache "
                    "between steps (warm cache); not the reported value",
            "ms": round(warm_ms, 5), "GB/s": round(one_bytes / (warm_ms * 1e-3) / 1e9, 1)}
    res["skip_ab"] = skip_ab(sets, args.steps, torch)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_grpo(case, old, level)
    return res


def skip_ab(sets, steps, torch, rounds=5):
    """The backward alone with its all-zero path (A) and with every row forced
    through the dense path (B), in interleaved A B B A rounds, as the Liger
    GRPO-backward analysis measures it ("Review feedback"); median of the
    per-round averages.  Outputs are identical either way (tested)."""
    a_ms, b_ms = [], []
    for _ in range(rounds):
        for which in ("bwd", "dense", "dense", "bwd"):
            (t,) = kernel_times([[s[which]] for s in sets], steps, torch)
            (a_ms if which == "bwd" else b_ms).append(t)
    a, b = float(np.median(a_ms)), float(np.median(b_ms))
    return {"rounds": rounds, "order": "ABBA", "skip_ms": round(a, 5), "dense_ms": round(b, 5),
            "speedup": round(b / a, 3), "time_saved_pct": round(100.0 * (1.0 - a / b), 1)}


def cpu_grpo(case, old, level):
    """The float64 oracle on the GRPO workload: whole steps for the headline,
    whole sequences for the sequence level, until about 10 s of CPU work."""
    import oracle
    B = case.B if level == "token" else 1
    R = B * case.L
    reps, t0 = 0, time.perf_counter()
    while True:
        z = oracle.decode_bf16(case.logits[:R])
        a = dict(z=z, ids=case.ids[:R], old_logp=old[:R].astype(np.float64), ref_logp=None,
                 adv=case.adv[:B], mask=case.mask[:R], B=B, L=case.L,
                 temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
                 eps_high=case.eps_high, level=level)
        fwd = oracle.grpo_forward(**a)
        dz, g, zr = oracle.grpo_backward(dloss=case.dloss[:R], fwd=fwd, **a)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 30:
            break
    dt = (time.perf_counter() - t0) / reps
    nz = int((~zr).sum())
    nbytes = R * case.V * 4 + nz * case.V * 2 + R * (FWD_ROW_BYTES + BWD_ROW_BYTES)
    what = "full steps" if level == "token" else "single sequences"
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} {what} (fwd+bwd, {R} rows x {case.V}) in float64 NumPy, "
                      f"{dt:.3f} s each, single thread; {R / dt:.0f} rows/s; host CPU {cpu_model()}"}


# ---------------------------------------------------------------------------
# entropy + selective log-softmax
# ---------------------------------------------------------------------------
def run_rows(args, torch, grl, synth):
    case = synth.row_case()
    N, V = case.N, case.V
    z = torch.from_numpy(case.logits.view(np.int16)).view(torch.bfloat16).cuda()
    if args.strided:
        buf = torch.empty((N, 2 * V), dtype=torch.bfloat16, device="cuda")
        buf[:, V:] = float("nan")
        buf[:, :V] = z
        del z
        z = buf[:, :V]
    ids = torch.from_numpy(case.ids).cuda()
    grad = torch.from_numpy(case.grad).cuda()
    H = torch.empty(N, device="cuda")
    lp = torch.empty(N, device="cuda")
    lse = torch.empty(N, device="cuda")
    dz = torch.empty((N, V), dtype=torch.bfloat16, device="cuda")
    L = grl.lib()
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ld = z.stride(0)

    def chk(st):
        if st != 0:
            raise grl.GrpoError("rows", st)
    f_ent = lambda: chk(L.entropy_from_logits(P(z), 1, N, V, ld, 1.0, P(H), s))
    f_lsm = lambda: chk(L.selective_log_softmax(P(z), 1, N, V, ld, P(ids), 1.0, P(lp), P(lse), s))
    f_bwd = lambda: chk(L.selective_log_softmax_bwd(P(z), 1, N, V, ld, P(ids), 1.0, P(lse), P(grad),
                                                    P(dz), V, s))
    launches = [f_ent, f_lsm, f_bwd]
    step = lambda: [f() for f in launches]
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 20))
    args.steps = steps
    ms = timed([step], steps, torch)
    kt = kernel_times([launches], steps, torch)
    kb = [N * V * 2, N * V * 2, 2 * N * V * 2]
    names = ["entropy", "lsm_fwd", "lsm_bwd"]
    step_bytes = sum(kb) + N * (4 + 8 + 8 + 8 + 4)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    k = int(np.argmax(kt))
    res = base_line(args, "entropy + selective log-softmax fwd+bwd GB/s at 65536x32000 bf16",
                    gbs, "GB/s", ms,
                    {"workload": "entropy_from_logits + selective_log_softmax fwd + bwd, N=65536 "
                                 "(B16 L4096) V=32000 bf16, N(0,3^2) + 8 peak" +
                                 (", rows of a [N, 2V] buffer" if args.strided else ""),
                     "rows": N, "V": V, "row_stride": ld})
    res.update({
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "kernels": {n: {"ms": round(t, 4), "GB/s": round(b / (t * 1e-3) / 1e9, 1)}
                    for n, t, b in zip(names, kt, kb)},
        "roofline": {"kernel": names[k], "bound": "hbm",
                     "achieved": round(kb[k] / (kt[k] * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kb[k] / (kt[k] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(names[k], "rows")},
    })
    if not args.no_cpu_baseline:
        import oracle
        R = 512
        reps, t0 = 0, time.perf_counter()
        while True:
            zz = oracle.decode_bf16(case.logits[:R])
            oracle.entropy_from_logits(zz)
            oracle.selective_log_softmax(zz, case.ids[:R])
            oracle.selective_log_softmax_bwd(zz, case.ids[:R], case.grad[:R])
            reps += 1
            if time.perf_counter() - t0 > 10.0 or reps >= 30:
                break
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": R * V * 8 / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} x {R} rows (entropy, selective fwd, bwd) in "
                                         f"float64 NumPy, {dt:.3f} s each, single thread; host "
                                         f"CPU {cpu_model()}"}
    return res


# ---------------------------------------------------------------------------
# steps either side of the row pass: entropy backward, advantages, weights
# ---------------------------------------------------------------------------
def run_entropy_bwd(args, torch, grl, synth):
    """entropy_from_logits_bwd over the rows workload's logits (lse and H from
    the forwards, upstream grad N(0, 1): every row dense), plus the latency
    of grpo_group_advantages and grpo_loss_weights at the headline's sizes."""
    case = synth.row_case()
    N, V = case.N, case.V
    z = torch.from_numpy(case.logits.view(np.int16)).view(torch.bfloat16).cuda()
    ids = torch.from_numpy(case.ids).cuda()
    grad = torch.from_numpy(case.grad).cuda()
    _, lse = grl.selective_log_softmax(z, ids)
    H = grl.entropy_from_logits(z)
    dz = torch.empty((N, V), dtype=torch.bfloat16, device="cuda")
    L = grl.lib()
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def chk(st):
        if st != 0:
            raise grl.GrpoError("entropy_from_logits_bwd", st)
    f_bwd = lambda: chk(L.entropy_from_logits_bwd(P(z), 1, N, V, V, 1.0, P(lse), P(H), P(grad),
                                                  P(dz), V, s))
    for _ in range(max(1, args.warmup)):
        f_bwd()
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 20))
    args.steps = steps
    ms = timed([f_bwd], steps, torch)
    (kt,) = kernel_times([[f_bwd]], steps, torch)
    n_nz = int((case.grad != 0).sum())
    nbytes = n_nz * V * 2 + N * V * 2 + N * 12
    gbs = nbytes / (ms * 1e-3) / 1e9
    kgbs = nbytes / (kt * 1e-3) / 1e9
    # the two small kernels, at the headline's B=4, L=512 (one group of 4)
    rewards = torch.tensor([1.0, 0.0, 1.0, 1.0], device="cuda")
    adv = torch.empty(4, device="cuda")
    mask = torch.from_numpy(synth.grpo_token_case(with_logits=False).mask).cuda()
    w = torch.empty(mask.numel(), device="cuda")
    f_adv = lambda: chk(L.grpo_group_advantages(P(rewards), 4, 4, 1e-4, 1, P(adv), s))
    f_w = lambda: chk(L.grpo_loss_weights(P(mask), 4, 512, 0, P(w), s))
    for f in (f_adv, f_w):
        f()
    t_adv, t_w = kernel_times([[f_adv, f_w]], 200, torch)
    res = base_line(args, "entropy backward GB/s at 65536x32000 bf16", gbs, "GB/s", ms,
                    {"workload": "entropy_from_logits_bwd, N=65536 V=32000 bf16, N(0,3^2) + 8 "
                                 "peak, upstream grad N(0,1) (no zero rows), T=1",
                     "rows": N, "V": V})
    res.update({
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "kernels": {"entropy_bwd": {"ms": round(kt, 4), "bytes": nbytes, "GB/s": round(kgbs, 1)},
                    "group_advantages_B4_G4": {"us": round(t_adv * 1e3, 2)},
                    "loss_weights_token_B4_L512": {"us": round(t_w * 1e3, 2)}},
        "roofline": {"kernel": "entropy_bwd", "bound": "hbm", "achieved": round(kgbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic("entropy_bwd", "entropy-bwd")},
    })
    if not args.no_cpu_baseline:
        import oracle
        R = 512
        reps, t0 = 0, time.perf_counter()
        while True:
            zz = oracle.decode_bf16(case.logits[:R])
            oracle.entropy_from_logits_bwd(zz, case.grad[:R])
            reps += 1
            if time.perf_counter() - t0 > 10.0 or reps >= 30:
                break
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": R * V * 4 / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} x {R} rows of the entropy backward in float64 "
                                         f"NumPy (computing lse and H itself), {dt:.3f} s each, "
                                         f"single thread; host CPU {cpu_model()}"}
    return res


# ---------------------------------------------------------------------------
# chunked fused-linear
# ---------------------------------------------------------------------------
def run_fused(args, torch, grl, synth):
    case = synth.fused_case(dloss="mean")
    rows = synth.stored_check_rows("fused")
    lp = synth.load_stored_logp("fused", case.hidden[rows])
    old = synth.add_noise_f32(lp, case.old_noise)
    ref = synth.add_noise_f32(lp, case.ref_noise)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    h = torch.from_numpy(case.hidden.view(np.int16)).view(torch.bfloat16).cuda()
    W = torch.from_numpy(case.weight.view(np.int16)).view(torch.bfloat16).cuda()
    ids, old_t, ref_t, adv, mask, dl = (dev(case.ids), dev(old), dev(ref), dev(case.adv),
                                        dev(case.mask), dev(case.dloss))
    c = args.chunk
    loss = torch.zeros(1, device="cuda")
    gW = torch.zeros((case.V, case.H), device="cuda")
    gh = torch.empty((case.N, case.H), device="cuda")
    ws = torch.empty(grl.fused_linear_grpo_workspace_bytes(c * case.L, case.V, case.H),
                     dtype=torch.uint8, device="cuda")
    kw = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
              eps_high=case.eps_high)
    calls = []
    for b0 in range(0, case.B, c):
        nb = min(c, case.B - b0)
        rs = slice(b0 * case.L, (b0 + nb) * case.L)
        calls.append(lambda rs=rs, b0=b0, nb=nb: grl.fused_linear_grpo_chunk(
            h[rs], W, ids[rs], old_t[rs], adv[b0:b0 + nb], mask[rs], dl[rs], nb, case.L,
            ref_logp=ref_t[rs], loss_accum=loss, grad_hidden=gh[rs], grad_weight=gW,
            workspace=ws, **kw))
    step = lambda: [f() for f in calls]
    for _ in range(max(1, min(args.warmup, 3))):
        step()
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 5))
    args.steps = steps
    base_bytes = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ms = timed([step], steps, torch)
    peak_bytes = torch.cuda.max_memory_allocated()
    # rows with dloss == 0 (padding) are compacted away before the products:
    # GEMM rates price the flops actually executed, on the kept rows
    kept = int((case.dloss != 0.0).sum())
    flops = 3 * 2.0 * kept * case.V * case.H
    tfs = flops / (ms * 1e-3) / 1e12
    dense_tfs = 3 * 2.0 * case.N * case.V * case.H / (ms * 1e-3) / 1e12
    rows_s = case.N / (ms * 1e-3)
    res = base_line(args, "chunked fused-linear GRPO fwd+bwd rows/s at B32 L1024 H1024 V151936 "
                          "bf16", rows_s, "rows/s", ms,
                    {"workload": f"fused-linear GRPO, h [32768, 1024] x W [151936, 1024] bf16, "
                                 f"{c} sequences per chunk, T=0.9 beta=0.04, lengths "
                                 f"U{{512..1024}}",
                     "chunk_sequences": c, "workspace_bytes": ws.numel(),
                     "full_logits_fp32_bytes": case.N * case.V * 4})
    # device memory while the batch runs: everything the caller holds (h, W,
    # inputs, grad_hidden, grad_weight, the workspace) and nothing the library
    # allocates; an unchunked loss would hold the batch's full logits besides
    res["memory"] = {"allocated_bytes": base_bytes, "peak_during_batch_bytes": peak_bytes,
                     "workspace_bytes": ws.numel(),
                     "full_logits_bf16_bytes": case.N * case.V * 2,
                     "full_logits_fp32_bytes": case.N * case.V * 4}
    # the dominant kernel, the logits product with its statistics epilogue,
    # timed alone on the first chunk's kept rows: back-to-back launches
    # between two events on the launch stream
    rows0 = torch.nonzero(dl[:c * case.L] != 0).flatten()
    h0 = h.index_select(0, rows0).contiguous()
    ids0 = ids.index_select(0, rows0).contiguous()
    rc0 = int(rows0.numel())
    z16 = torch.empty((rc0, case.V), dtype=torch.bfloat16, device="cuda")
    st0 = torch.empty((2, grl.logits_partials(case.V), rc0), dtype=torch.float32, device="cuda")
    zy0 = torch.empty(rc0, dtype=torch.float32, device="cuda")
    logits = lambda: grl.grpo_gemm_bf16_logits(h0, W, ids0, temperature=case.temperature,
                                               z16=z16, stat=st0, zy=zy0)
    for _ in range(3):
        logits()
    kms = kernel_times([[logits]], 20, torch)[0]
    ktf = 2.0 * rc0 * case.V * case.H / (kms * 1e-3) / 1e12
    del z16, st0, zy0
    res.update({
        "rows_kept": kept, "rows_total": case.N,
        "gemm_tflops_executed": round(tfs, 1),
        "gemm_tflops_dense_equivalent": round(dense_tfs, 1),
        "pct_mfma_peak": round(100.0 * tfs / MFMA_BF16_PEAK_TFS, 2),
        "kernels": {"logits_product": {"ms": round(kms, 4), "rows": rc0,
                                       "TFLOP/s": round(ktf, 1)}},
        "roofline": {"kernel": f"logits product with row statistics (grpo_gemm_bf16_logits, "
                               f"the first chunk's {rc0} kept rows x V x H)",
                     "bound": "mfma", "achieved": round(ktf, 1), "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(ktf / MFMA_BF16_PEAK_TFS, 4),
                     "traffic": None},
    })
    # per-product MFMA utilisation and rate from the stored rocprofv3 runs (4-sequence chunks)
    stored = stored_counters("fused-linear")
    gem = {k: v for k, v in stored.items() if "mfma_util" in v}
    if gem and c == 4:
        res["gemm_counters"] = {k: {"mfma_util": v["mfma_util"], "trace_avg_us": v["trace_avg_us"],
                                    "TFLOP/s": v["tflops"]} for k, v in gem.items()}
        # dz W and dz^T h run side by side: their trace durations overlap, the
        # pair's span per chunk is the figure that adds up
        pair = stored.get("gradient pair")
        if pair:
            res["gemm_counters"]["gradient pair (concurrent)"] = {
                "span_us": pair["span_us"], "TFLOP/s": pair["tflops"]}
    if not args.no_cpu_baseline:
        import oracle
        hh = oracle.decode_bf16(case.hidden[:case.L])
        WW = oracle.decode_bf16(case.weight)
        t0 = time.perf_counter()
        oracle.fused_linear_grpo(hh, WW, case.ids[:case.L], old[:case.L].astype(np.float64),
                                 ref[:case.L].astype(np.float64), case.adv[:1],
                                 case.mask[:case.L], case.dloss[:case.L], 1, case.L,
                                 case.temperature, case.beta, case.eps_low, case.eps_high, 1)
        dt = time.perf_counter() - t0
        cores = len(os.sched_getaffinity(0))
        res["cpu_baseline"] = {"value": case.L / dt, "unit": "rows/s", "cores": cores,
                               "kind": "oracle",
                               "sample": f"one sequence (1024 rows, every row computed) of the "
                                         f"fused-linear loss in float64 NumPy/BLAS, {dt:.2f} s "
                                         f"= {3 * 2.0 * case.L * case.V * case.H / dt / 1e12:.3f}"
                                         f" TFLOP/s; up to {cores} BLAS threads; host CPU "
                                         f"{cpu_model()}"}
    return res


# ---------------------------------------------------------------------------
# tiny GRPO case (latency)
# ---------------------------------------------------------------------------
def run_tiny(args, torch, grl, synth):
    """B=2 L=16 V=1024 fp32 logits, beta 0.04 with a reference, sequence 1 at
    advantage 0: one fwd+bwd step is a few microseconds of launch latency,
    reported as time.  The step is the single pass; the two-pass step is
    timed beside it."""
    case = synth.tiny_case("a")
    logp_true = synth.load_stored_logp("tiny", case.logits[synth.stored_check_rows("tiny")])
    old = synth.add_noise_f32(logp_true, case.old_noise)
    ref = synth.add_noise_f32(logp_true, case.ref_noise)
    B, L, V, N = case.B, case.L, case.V, case.N
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    z, ids, old_t, ref_t, adv, mask, dloss = (dev(case.logits), dev(case.ids), dev(old), dev(ref),
                                              dev(case.adv), dev(case.mask), dev(case.dloss))
    kw = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
              eps_high=case.eps_high)
    dz = torch.empty((N, V), dtype=torch.float32, device="cuda")
    zr = torch.empty(N, dtype=torch.uint8, device="cuda")
    one, _, _, _ = grl.grpo_logits_fwd_bwd(z, ids, old_t, adv, B, L, dloss, ref_logp=ref_t,
                                           mask=mask, dlogits=dz, zero_row=zr, prepare=True,
                                           **kw)
    fwd, out2 = grl.grpo_logits_fwd(z, ids, old_t, adv, B, L, ref_logp=ref_t, mask=mask,
                                    prepare=True, **kw)
    bwd, _, _ = grl.grpo_logits_bwd(z, ids, old_t, adv, B, L, out2["logp"], out2["lse"], dloss,
                                    ref_logp=ref_t, mask=mask, dlogits=dz, zero_row=zr,
                                    prepare=True, **kw)
    for _ in range(args.warmup):
        one()
        fwd()
        bwd()
    torch.cuda.synchronize()
    ms = timed([one], args.steps, torch)
    (one_ms,) = kernel_times([[one]], args.steps, torch)
    ms_two = timed([lambda: (fwd(), bwd())], args.steps, torch)
    one()
    torch.cuda.synchronize()
    n_zero = int(zr.sum().item())
    step_bytes = 2 * N * V * 4 + N * ONE_ROW_BYTES
    gbs = step_bytes / (one_ms * 1e-3) / 1e9
    res = base_line(args, "tiny GRPO loss fwd+bwd latency at B2 L16 V1024 fp32", ms * 1e3, "us",
                    ms, {"workload": "token-level GRPO fwd+bwd in one pass, B=2 L=16 V=1024 fp32 "
                                     "(T=1, beta=0.04 with a reference, eps 0.2/0.2, sequence 1 "
                                     "at advantage 0, sum dloss)", "rows": N, "V": V,
                         "zero_rows": n_zero, "accumulate": "fp32"}, dtype="f32")
    res.update({
        "higher_is_better": False,
        "rows_per_s": round(N / (ms * 1e-3), 1),
        "two_pass_us": round(ms_two * 1e3, 2),
        "kernels": {"grpo_fwd_bwd": {"ms": round(one_ms, 5), "bytes": step_bytes,
                                     "GB/s": round(gbs, 1)}},
        "roofline": {"kernel": "grpo_fwd_bwd (launch-latency bound at 256 KiB)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    })
    if not args.no_cpu_baseline:
        import oracle
        a = dict(z=case.logits.astype(np.float64), ids=case.ids, old_logp=old.astype(np.float64),
                 ref_logp=ref.astype(np.float64), adv=case.adv, mask=case.mask, B=B, L=L,
                 temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
                 eps_high=case.eps_high, level="token")
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0 and reps < 20000:
            f = oracle.grpo_forward(**a)
            oracle.grpo_backward(dloss=case.dloss, fwd=f, **a)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": round(dt * 1e6, 1), "unit": "us", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} full steps (fwd+bwd, {N} rows x {V}) in float64 "
                                         f"NumPy, single thread; host CPU {cpu_model()}"}
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (the row "
              "pass would shard by sequence with no exchange; the fused-linear path would "
              "all-reduce grad_weight once per step).", file=sys.stderr)
        sys.exit(2)
    import torch
    import rl_fine_tuning_row_amd as grl
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    grl.lib()  # raises if the HIP library is missing
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.workload == "grpo-token":
        res = run_grpo(args, torch, grl, synth, "token")
    elif args.workload == "grpo-seq":
        res = run_grpo(args, torch, grl, synth, "sequence")
    elif args.workload == "rows":
        res = run_rows(args, torch, grl, synth)
    elif args.workload == "entropy-bwd":
        res = run_entropy_bwd(args, torch, grl, synth)
    elif args.workload == "tiny":
        res = run_tiny(args, torch, grl, synth)
    else:
        res = run_fused(args, torch, grl, synth)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
