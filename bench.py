"""Benchmark of the GRPO logits row pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--sets S] [--chunk C] [--no-cpu-baseline] [--no-configs]
                    [--copy-probe]

Default workload ``grpo-token`` (the headline): a step is one forward +
backward of the token-level GRPO loss over the logits of B=4 sequences x
L=512 tokens x V=32000 vocabulary entries (bf16, T=0.9, beta=0.04, eps
0.2/0.28, half the advantages exactly 0, no reference model so the KL term
vanishes, token-mean upstream gradient), run as the single pass
grpo_logits_fwd_bwd: loss, logp, lse, entropy, kl and is_clipped per token
and dlogits (all-zero rows where dlogp is 0) from one read of the logits.
The two-pass step (grpo_logits_fwd then grpo_logits_bwd) is timed too and
reported under "two_pass", and the same steps with a reference model
(ref = logp + N(0, 0.1^2): every kept row carries the KL gradient) under
"with_reference".  S buffer sets (about 1 GB in total by default) rotate
from step to step so a step does not find the previous step's logits in the
256 MB last-level cache.

The default run also measures the other workloads, each with a bounded
number of steps, and reports them in the same line under "configs" (the
headline's value is unchanged by them; --no-configs skips them):
  grpo-seq      sequence-level fwd+bwd, B=8 L=1024 V=151936 bf16, beta=0
  rows          entropy_from_logits + selective_log_softmax fwd + bwd,
                65536 x 32000 bf16 (contiguous; rows-strided: rows of a 2V
                buffer), with the device memory the calls allocate
  entropy-bwd   entropy_from_logits_bwd over the rows workload's logits,
                plus the latency of grpo_group_advantages / grpo_loss_weights
  fused-linear  chunked fused-linear loss over h [32768, 1024] and
                W [151936, 1024] bf16, --chunk sequences per call (value:
                rows/s; roofline on the dominant kernel, the logits product
                with its row statistics, timed alone on the first chunk's
                kept rows; zero-weight rows are skipped), with the device
                peak of the chunked batch beside the library's own unchunked
                composition of the same loss
  tiny          the B=2 L=16 V=1024 fp32 GRPO step (value: microseconds per
                step, lower is better; launch-latency bound)
``--workload NAME`` runs one of them alone and prints its own line.

Inputs are synthetic, generated on the host and already resident in device
memory when the timed region starts; the per-token weights dloss of the
token-mean reduction come from the library's grpo_loss_weights.  ``value``
is GB/s of algorithmic HBM bytes (rows/s for fused-linear) over the wall time
of the timed steps.  ``roofline`` is for the step's dominant kernel, its
duration timed with events on the launch stream over back-to-back launches;
``traffic`` is the HBM bytes per launch from rocprofv3 FETCH_SIZE /
WRITE_SIZE counters stored in profiles/counters.json, used only while the
kernels' source digest matches.  ``cpu_baseline`` times the float64 oracle on
a bounded sample of the same workload on the host's cores: a pool of
processes (one BLAS thread each, forked before any GPU call) over blocks of
rows, or, for the fused-linear loss, NumPy's BLAS on every core.
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
    ap.add_argument("--no-reference", action="store_true",
                    help="grpo-token: skip the with-reference reading's timing (profiling runs)")
    ap.add_argument("--no-unchunked", action="store_true",
                    help="fused-linear: skip the unchunked composition's memory comparison")
    ap.add_argument("--no-configs", action="store_true",
                    help="default workload only: skip the other workloads' measurements")
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


# GPU-side spin (torch's own sleep kernel) queued after the synchronize that
# opens a timed region and before its start event: while the GPU spins, the
# host enqueues the first launches of the region, so the region measures the
# steps back to back rather than the host's latency in issuing the first one.
GATE_CYCLES = 200_000


def gate(torch):
    torch.cuda._sleep(GATE_CYCLES)


def timed(step_fns, steps, torch):
    """Wall time (ms) per step of `steps` steps rotating over step_fns,
    between two events on the launch stream (opened behind the gate)."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gate(torch)
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
        gate(torch)
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


# ---------------------------------------------------------------------------
# the oracle on the host's cores
# ---------------------------------------------------------------------------
_POOL = None
_POOL_SIZE = 1
_THREAD_LIMIT = None


def _worker_init():
    """One BLAS / OpenMP thread per worker process."""
    global _THREAD_LIMIT
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        _THREAD_LIMIT = threadpool_limits(1)
    except ImportError:
        pass


def start_pool():
    """Fork the oracle's worker pool: before any GPU call, so no worker
    inherits an initialised GPU runtime.  One worker per core of the
    process's CPU share, at most 16 (one GPU's share of the host)."""
    global _POOL, _POOL_SIZE
    import multiprocessing as mp
    _POOL_SIZE = max(1, min(16, len(os.sched_getaffinity(0))))
    _POOL = mp.get_context("fork").Pool(_POOL_SIZE, initializer=_worker_init)


def stop_pool():
    if _POOL is not None:
        _POOL.close()
        _POOL.join()


def pool_run(fn, tasks):
    """Wall time (s) of fn over the tasks on the pool (or inline without one)."""
    t0 = time.perf_counter()
    if _POOL is None:
        for t in tasks:
            fn(t)
    else:
        _POOL.map(fn, tasks, chunksize=1)
    return time.perf_counter() - t0


def _oracle_grpo_task(t):
    """Oracle forward + backward of one block of GRPO rows (whole sequences)."""
    import oracle
    (bits, dtype, ids, old, ref, adv, mask, dloss, B, L, T, beta, el, eh, level) = t
    z = oracle.decode_bf16(bits) if dtype == "bf16" else bits.astype(np.float64)
    a = dict(z=z, ids=ids, old_logp=old, ref_logp=ref, adv=adv, mask=mask, B=B, L=L,
             temperature=T, beta=beta, eps_low=el, eps_high=eh, level=level)
    fwd = oracle.grpo_forward(**a)
    oracle.grpo_backward(dloss=dloss, fwd=fwd, **a)
    return B * L


def _oracle_grpo_reps_task(t):
    """`reps` oracle steps of one GRPO task (for steps far below a task's overhead)."""
    reps, task = t
    for _ in range(reps):
        _oracle_grpo_task(task)
    return reps


def _oracle_rows_task(t):
    """Oracle entropy, selective log-softmax and its backward on a block of rows."""
    import oracle
    bits, ids, grad = t
    z = oracle.decode_bf16(bits)
    oracle.entropy_from_logits(z)
    oracle.selective_log_softmax(z, ids)
    oracle.selective_log_softmax_bwd(z, ids, grad)
    return z.shape[0]


def _oracle_entropy_bwd_task(t):
    import oracle
    bits, grad = t
    oracle.entropy_from_logits_bwd(oracle.decode_bf16(bits), grad)
    return bits.shape[0]


def cpu_entry(value, unit, sample, dt_wall, work_rows=None):
    d = {"value": value, "unit": unit, "cores": _POOL_SIZE, "kind": "oracle",
         "sample": f"{sample}; {dt_wall:.2f} s wall on {_POOL_SIZE} worker processes "
                   f"(one BLAS thread each); host CPU {cpu_model()}"}
    if work_rows is not None:
        d["rows_per_s"] = round(work_rows / dt_wall, 1)
    return d


def grpo_row_tasks(case, bits, old, ref, dloss, level, block_rows=128):
    """Oracle tasks over one step's rows: token level in blocks of rows (each
    row its own unit: B = rows, L = 1, advantage per row); sequence level in
    whole sequences."""
    N = case.N
    A_row = np.repeat(case.adv.astype(np.float64), case.L)
    tasks = []
    if level == "token":
        for r0 in range(0, N, block_rows):
            rs = slice(r0, min(N, r0 + block_rows))
            n = rs.stop - rs.start
            tasks.append((bits[rs], case.dtype, case.ids[rs], old[rs].astype(np.float64),
                          None if ref is None else ref[rs].astype(np.float64), A_row[rs],
                          case.mask[rs], dloss[rs], n, 1, case.temperature, case.beta,
                          case.eps_low, case.eps_high, "token"))
    else:
        for b in range(case.B):
            rs = slice(b * case.L, (b + 1) * case.L)
            tasks.append((bits[rs], case.dtype, case.ids[rs], old[rs].astype(np.float64),
                          None if ref is None else ref[rs].astype(np.float64), case.adv[b:b + 1],
                          case.mask[rs], dloss[rs], 1, case.L, case.temperature, case.beta,
                          case.eps_low, case.eps_high, "sequence"))
    return tasks


def token_weights(torch, grl, mask_t, B, L):
    """dloss of the token-mean reduction, from the library."""
    return grl.grpo_loss_weights(mask_t, B, L, "token")


def oracle_token_weights(case):
    import oracle
    return oracle.loss_weights(case.mask, case.B, case.L, "token")


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
    "two_pass", and both again with a reference model under
    "with_reference".  Sequence level (needs the per-sequence ratio before any
    gradient): the two-pass step."""
    if level == "token":
        case = synth.grpo_token_case(with_ref=True, dloss="mean")
        name = "token"
    else:
        case = synth.grpo_sequence_case(dloss="mean")
        name = "sequence"
    logp_true = synth.load_stored_logp(name, case.logits[synth.stored_check_rows(name)])
    old = synth.add_noise_f32(logp_true, case.old_noise)
    ref = synth.add_noise_f32(logp_true, case.ref_noise) if case.ref_noise is not None else None
    B, L, V, N = case.B, case.L, case.V, case.N
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    z0 = torch.from_numpy(case.logits.view(np.int16)).view(torch.bfloat16).cuda()
    ids, old_t, adv, mask = dev(case.ids), dev(old), dev(case.adv), dev(case.mask)
    ref_t = dev(ref) if ref is not None else None
    dloss = token_weights(torch, grl, mask, B, L)
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
        entry = dict(zr=zr)
        # the primary reading (no reference model), and with a reference model
        for tag, rt in (("", None), ("ref_", ref_t)):
            if tag and (level != "token" or rt is None):
                continue
            # arguments marshalled once; a step is one (single pass) or two C calls
            fwd, out = grl.grpo_logits_fwd(z, ids, old_t, adv, B, L, ref_logp=rt, mask=mask,
                                           out=out, prepare=True, level=level, **kw)
            bwd, _, _ = grl.grpo_logits_bwd(z, ids, old_t, adv, B, L, out["logp"], out["lse"],
                                            dloss, ref_logp=rt, mask=mask,
                                            seq_ratio=out.get("seq_ratio"), dlogits=dz,
                                            zero_row=zr, prepare=True, level=level, **kw)
            entry[tag + "fwd"], entry[tag + "bwd"] = fwd, bwd
            if not tag:
                # the backward with the all-zero path switched off, for the skip A/B
                entry["dense"], _, _ = grl.grpo_logits_bwd(
                    z, ids, old_t, adv, B, L, out["logp"], out["lse"], dloss, mask=mask,
                    seq_ratio=out.get("seq_ratio"), dlogits=dz, zero_row=zr, prepare=True,
                    level=level, force_dense=True, **kw)
            if level == "token":
                entry[tag + "one"], _, _, _ = grl.grpo_logits_fwd_bwd(
                    z, ids, old_t, adv, B, L, dloss, ref_logp=rt, mask=mask, out=out,
                    dlogits=dz, zero_row=zr, prepare=True, **kw)
        sets.append(entry)
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
    one_bytes = 2 * N * V * 2 + N * ONE_ROW_BYTES
    if level == "token":
        # single pass: logits read once, dlogits written once
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
    if level == "token" and ref is not None and not args.no_reference:
        res["with_reference"] = with_reference(sets, args.steps, torch, N, V)
    if not args.no_cpu_baseline:
        w = oracle_token_weights(case)
        res["cpu_baseline"] = cpu_grpo(case, old, None, w, level,
                                       step_bytes if level == "token" else two_bytes)
    return res


def with_reference(sets, steps, torch, N, V):
    """The headline's steps with a reference model, ref_logp = logp + N(0, 0.1^2)
    (the other reading of the workload): the KL gradient makes every kept row
    dense, so only the masked (padding) rows stay zero."""
    for s in sets:
        s["ref_one"]()
        s["ref_fwd"]()
        s["ref_bwd"]()
    torch.cuda.synchronize()
    n_zero = int(sets[0]["zr"].sum().item())
    n_nz = N - n_zero
    one_bytes = 2 * N * V * 2 + N * ONE_ROW_BYTES
    fwd_bytes = N * V * 2 + N * FWD_ROW_BYTES + N * 4
    bwd_bytes = N * V * 2 + n_nz * V * 2 + N * BWD_ROW_BYTES + N * 4
    ms = timed([s["ref_one"] for s in sets], steps, torch)
    ms_two = timed([(lambda s=s: (s["ref_fwd"](), s["ref_bwd"]())) for s in sets], steps, torch)
    (one_ms,) = kernel_times([[s["ref_one"]] for s in sets], steps, torch)
    return {"reading": "ref_logp = logp + N(0, 0.1^2) (reference model present)",
            "zero_rows": n_zero, "nonzero_rows": n_nz,
            "zero_row_fraction": round(n_zero / N, 4),
            "single_pass": {"ms_per_step": round(ms, 5), "step_bytes": one_bytes,
                            "GB/s": round(one_bytes / (ms * 1e-3) / 1e9, 1),
                            "pct_hbm_peak": round(100.0 * one_bytes / (ms * 1e-3) / 1e9
                                                  / HBM_PEAK_GBS, 2),
                            "kernel_ms": round(one_ms, 5),
                            "rows_per_s": round(N / (ms * 1e-3), 1)},
            "two_pass": {"ms_per_step": round(ms_two, 5),
                         "step_bytes": fwd_bytes + bwd_bytes,
                         "GB/s": round((fwd_bytes + bwd_bytes) / (ms_two * 1e-3) / 1e9, 1),
                         "rows_per_s": round(N / (ms_two * 1e-3), 1)}}


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


def cpu_grpo(case, old, ref, dloss, level, step_bytes):
    """The float64 oracle's forward + backward of whole steps (the headline's
    2048 rows in blocks of 128, or the sequence level's eight sequences), on
    the worker pool, for about 10-30 core-seconds; GB/s with the GPU step's
    algorithmic bytes."""
    reps = 24 if level == "token" else 2
    tasks = grpo_row_tasks(case, case.logits, old, ref, dloss, level) * reps
    dt = pool_run(_oracle_grpo_task, tasks)
    per_step = dt / reps
    what = (f"{reps} full steps ({case.N} rows x {case.V}, fwd+bwd, blocks of 128 rows)"
            if level == "token" else
            f"{reps} full steps ({case.B} sequences of {case.L} rows x {case.V}, fwd+bwd, one "
            f"sequence per task)")
    return cpu_entry(round(step_bytes / per_step / 1e9, 3), "GB/s",
                     f"{what} in float64 NumPy, {per_step:.3f} s per step; GB/s with the GPU "
                     f"step's {step_bytes} algorithmic bytes", dt, reps * case.N)


# ---------------------------------------------------------------------------
# entropy + selective log-softmax
# ---------------------------------------------------------------------------
_ROW_CASE = None


def row_case(synth):
    """The 65536 x 32000 rows workload, generated once per run."""
    global _ROW_CASE
    if _ROW_CASE is None:
        _ROW_CASE = synth.row_case()
    return _ROW_CASE


def run_rows(args, torch, grl, synth, strided=None):
    strided = args.strided if strided is None else strided
    case = row_case(synth)
    N, V = case.N, case.V
    z = torch.from_numpy(case.logits.view(np.int16)).view(torch.bfloat16).cuda()
    if strided:
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
    # device memory the three calls allocate beyond their inputs and outputs
    # (all preallocated above): the allocator's live and peak bytes around them
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    step()
    torch.cuda.synchronize()
    mem = {"allocated_before_bytes": before,
           "allocated_after_bytes": torch.cuda.memory_allocated(),
           "peak_during_calls_bytes": torch.cuda.max_memory_allocated(),
           "extra_bytes": torch.cuda.max_memory_allocated() - before,
           "note": "the library allocates nothing: no temporary beyond the outputs (the pages "
                   "report >100 MB -> <10 MB of overhead for the chunked PyTorch entropy "
                   "against their kernel)"}
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    steps = max(1, min(args.steps, 20))
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
                                 (", rows of a [N, 2V] buffer" if strided else ""),
                     "rows": N, "V": V, "row_stride": ld})
    res["steps"] = steps
    res.update({
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "step_bytes": step_bytes,
        "memory": mem,
        "kernels": {n: {"ms": round(t, 4), "GB/s": round(b / (t * 1e-3) / 1e9, 1)}
                    for n, t, b in zip(names, kt, kb)},
        "roofline": {"kernel": names[k], "bound": "hbm",
                     "achieved": round(kb[k] / (kt[k] * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kb[k] / (kt[k] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(names[k], "rows")},
    })
    if not args.no_cpu_baseline and not strided:
        R, nblk = 512, 64
        tasks = [(case.logits[b * R:(b + 1) * R], case.ids[b * R:(b + 1) * R],
                  case.grad[b * R:(b + 1) * R].astype(np.float64)) for b in range(nblk)]
        dt = pool_run(_oracle_rows_task, tasks)
        rows = R * nblk
        res["cpu_baseline"] = cpu_entry(
            round(step_bytes * rows / N / dt / 1e9, 3), "GB/s",
            f"{rows} of the {N} rows in blocks of {R} (entropy, selective fwd, bwd) in float64 "
            f"NumPy; GB/s with the GPU step's algorithmic bytes per row", dt, rows)
    del z, dz
    return res


# ---------------------------------------------------------------------------
# steps either side of the row pass: entropy backward, advantages, weights
# ---------------------------------------------------------------------------
def run_entropy_bwd(args, torch, grl, synth):
    """entropy_from_logits_bwd over the rows workload's logits (lse and H from
    the forwards, upstream grad N(0, 1): every row dense), plus the latency
    of grpo_group_advantages and grpo_loss_weights at the headline's sizes."""
    case = row_case(synth)
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
    res["steps"] = steps
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
        R, nblk = 512, 128
        tasks = [(case.logits[b * R:(b + 1) * R], case.grad[b * R:(b + 1) * R].astype(np.float64))
                 for b in range(nblk)]
        dt = pool_run(_oracle_entropy_bwd_task, tasks)
        rows = R * nblk
        res["cpu_baseline"] = cpu_entry(
            round(nbytes * rows / N / dt / 1e9, 3), "GB/s",
            f"{rows} rows in blocks of {R} of the entropy backward in float64 NumPy (lse and H "
            f"computed by the oracle itself); GB/s with the GPU kernel's algorithmic bytes per "
            f"row", dt, rows)
    del z, dz
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
    ids, old_t, ref_t, adv, mask = (dev(case.ids), dev(old), dev(ref), dev(case.adv),
                                    dev(case.mask))
    dl = token_weights(torch, grl, mask, case.B, case.L)
    c = args.chunk
    loss = torch.zeros(1, device="cuda")
    gW = torch.zeros((case.V, case.H), device="cuda")
    gh = torch.empty((case.N, case.H), device="cuda")
    kw = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
              eps_high=case.eps_high)
    torch.cuda.synchronize()
    base_bytes = torch.cuda.memory_allocated()  # inputs, weights, gradients: held either way
    torch.cuda.reset_peak_memory_stats()
    ws = torch.empty(grl.fused_linear_grpo_workspace_bytes(c * case.L, case.V, case.H),
                     dtype=torch.uint8, device="cuda")
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
    ms = timed([step], steps, torch)
    peak_chunked = torch.cuda.max_memory_allocated()
    # rows with dloss == 0 (padding) are compacted away before the products:
    # GEMM rates price the flops actually executed, on the kept rows
    kept = int((case.mask != 0).sum())
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
    res["steps"] = steps
    del ws
    torch.cuda.empty_cache()
    if not args.no_unchunked:
        res["memory"] = fused_memory(torch, grl, case, h, W, ids, old_t, ref_t, adv, mask, dl,
                                     kw, base_bytes, peak_chunked, ms)
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
        res["cpu_baseline"] = cpu_fused(case, old, ref)
    return res


def fused_memory(torch, grl, case, h, W, ids, old_t, ref_t, adv, mask, dl, kw, base_bytes,
                 peak_chunked, ms_chunked):
    """Device memory of the chunked batch against the library's own unchunked
    composition of the same loss (the whole batch's logits at once: the logits
    product to bf16, the two-pass row forward and in-place backward over them,
    then the two gradient products), both measured with the allocator over
    one batch from the same resident inputs (the unchunked run starts after
    the chunked one has released its workspace)."""
    B, L, V, H, N = case.B, case.L, case.V, case.H, case.N
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    t0 = time.perf_counter()
    z16, _, _ = grl.grpo_gemm_bf16_logits(h, W, ids, temperature=case.temperature)
    fwd = grl.grpo_logits_fwd(z16, ids, old_t, adv, B, L, ref_logp=ref_t, mask=mask,
                              entropy=False, kl=False, is_clipped=False, **kw)
    grl.grpo_logits_bwd(z16, ids, old_t, adv, B, L, fwd["logp"], fwd["lse"], dl,
                        ref_logp=ref_t, mask=mask, dlogits=z16, zero_row=False, **kw)
    gh = grl.grpo_gemm_bf16(z16, W, a_layout=0, b_layout=1)
    gW = torch.zeros((V, H), device="cuda")
    grl.grpo_gemm_bf16(z16, h, a_layout=1, b_layout=1, C=gW, accumulate=True)
    torch.cuda.synchronize()
    ms_unchunked = (time.perf_counter() - t0) * 1e3
    peak_unchunked = torch.cuda.max_memory_allocated()
    del z16, fwd, gh, gW
    torch.cuda.empty_cache()
    return {"inputs_and_gradients_bytes": base_bytes,
            "peak_chunked_bytes": peak_chunked,
            "peak_unchunked_bytes": peak_unchunked,
            "peak_reduction_pct": round(100.0 * (1.0 - peak_chunked / peak_unchunked), 1),
            "chunked_batch_ms": round(ms_chunked, 3),
            "unchunked_batch_ms_first_run": round(ms_unchunked, 3),
            "full_logits_bf16_bytes": N * V * 2,
            "full_logits_fp32_bytes": N * V * 4,
            "note": "unchunked: full-batch logits product (bf16 logits + row statistics), "
                    "grpo_logits_fwd and in-place grpo_logits_bwd over them, grpo_gemm_bf16 for "
                    "both gradients (every row computed: no zero-row compaction); one cold run, "
                    "host-timed, for context only"}


def cpu_fused(case, old, ref):
    """The float64 oracle's chunked loss on one 1024-row sequence (every row
    computed), its products in NumPy's BLAS on every core of the process's
    share (the row work there is a small part)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(_POOL_SIZE)
    except ImportError:
        limit = None
    w = oracle_token_weights(case)
    hh = oracle.decode_bf16(case.hidden[:case.L])
    WW = oracle.decode_bf16(case.weight)
    t0 = time.perf_counter()
    oracle.fused_linear_grpo(hh, WW, case.ids[:case.L], old[:case.L].astype(np.float64),
                             ref[:case.L].astype(np.float64), case.adv[:1], case.mask[:case.L],
                             w[:case.L], 1, case.L, case.temperature, case.beta, case.eps_low,
                             case.eps_high, 1)
    dt = time.perf_counter() - t0
    if limit is not None:
        limit.restore_original_limits()
    return {"value": round(case.L / dt, 1), "unit": "rows/s", "cores": _POOL_SIZE,
            "kind": "oracle",
            "sample": f"one sequence (1024 rows, every row computed) of the fused-linear loss in "
                      f"float64 NumPy, {dt:.2f} s = "
                      f"{3 * 2.0 * case.L * case.V * case.H / dt / 1e12:.3f} TFLOP/s; "
                      f"{_POOL_SIZE} BLAS threads; host CPU {cpu_model()}"}


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
    z, ids, old_t, ref_t, adv, mask = (dev(case.logits), dev(case.ids), dev(old), dev(ref),
                                       dev(case.adv), dev(case.mask))
    dloss = token_weights(torch, grl, mask, B, L)
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
                                     "at advantage 0, token-mean dloss)", "rows": N, "V": V,
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
        w = oracle_token_weights(case)
        per_task, ntasks = 3000, _POOL_SIZE
        steps_cpu = per_task * ntasks
        task = (case.logits, "f32", case.ids, old.astype(np.float64), ref.astype(np.float64),
                case.adv, case.mask, w, B, L, case.temperature, case.beta, case.eps_low,
                case.eps_high, "token")
        dt = pool_run(_oracle_grpo_reps_task, [(per_task, task)] * ntasks)
        res["cpu_baseline"] = cpu_entry(
            round(dt / steps_cpu * 1e6, 2), "us",
            f"{steps_cpu} full steps (fwd+bwd, {N} rows x {V}) in float64 NumPy, {per_task} "
            f"steps per task; value = wall time / steps (several steps in flight at once, so a "
            f"throughput figure, not one step's latency)", dt, steps_cpu * N)
    return res


def compact(res):
    """A workload's line without the fields the headline line already carries."""
    return {k: v for k, v in res.items() if k not in ("n_gpus", "scaling", "vs_baseline", "data")}


def progress(msg, t0):
    print(f"[bench] {msg} ({time.perf_counter() - t0:.0f} s)", file=sys.stderr, flush=True)


def run_configs(args, torch, grl, synth, t0):
    """The other workloads, each with its own bounded steps, for the headline
    line's "configs" object."""
    out = {}
    jobs = [("tiny", lambda a: run_tiny(a, torch, grl, synth)),
            ("grpo-seq", lambda a: run_grpo(a, torch, grl, synth, "sequence")),
            ("rows", lambda a: run_rows(a, torch, grl, synth, strided=False)),
            ("rows-strided", lambda a: run_rows(a, torch, grl, synth, strided=True)),
            ("entropy-bwd", lambda a: run_entropy_bwd(a, torch, grl, synth)),
            ("fused-linear", lambda a: run_fused(a, torch, grl, synth))]
    for name, fn in jobs:
        sub = argparse.Namespace(**vars(args))
        sub.steps = min(args.steps, 200)
        sub.warmup = min(max(args.warmup, 1), 20)
        sub.chunk = 4
        out[name] = compact(fn(sub))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        progress(f"{name} done", t0)
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (the row "
              "pass would shard by sequence with no exchange; the fused-linear path would "
              "all-reduce grad_weight once per step).", file=sys.stderr)
        sys.exit(2)
    t0 = time.perf_counter()
    if not args.no_cpu_baseline and not args.copy_probe:
        start_pool()  # before the first GPU call
    import torch
    import rl_fine_tuning_row_amd as grl
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    grl.lib()  # raises if the HIP library is missing
    try:
        if args.copy_probe:
            copy_probe(torch)
            return
        if args.workload == "grpo-token":
            res = run_grpo(args, torch, grl, synth, "token")
            progress("headline done", t0)
            if not args.no_configs:
                torch.cuda.empty_cache()
                res["configs"] = run_configs(args, torch, grl, synth, t0)
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
    finally:
        stop_pool()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
