"""Benchmark of the GRPO logits row pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sets S] [--no-cpu-baseline]

A step is one forward + backward of the token-level GRPO loss over the
logits of B=4 sequences x L=512 tokens x V=32000 vocabulary entries (bf16,
T=0.9, beta=0.04, eps 0.2/0.28, half the advantages exactly 0, no reference
model so the KL term vanishes, token-mean upstream gradient):
grpo_logits_fwd writes loss, logp, lse, entropy, kl and is_clipped per token;
grpo_logits_bwd writes dlogits with the all-zero path on rows whose dlogp is 0.
Inputs are synthetic and already resident in device memory; S input/output
buffer sets (about 1 GB in total by default) rotate from step to step so a
step does not find the previous step's logits in the 256 MB last-level cache.

Prints one JSON line.  `value` is GB/s of algorithmic HBM bytes (logits read
by the forward, logits re-read by the backward on its non-zero rows, dlogits
written, plus the per-row scalars) over the wall time of the timed steps.
`roofline` is for the dominant kernel, timed with events on its stream.
`cpu_baseline` times the float64 oracle on the same workload on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of 256 MiB (counter calibration)")
    return ap.parse_args()


def per_row_bytes_fwd():
    # ids int64, old_logp f32, adv (per sequence, negligible); out: loss, logp,
    # lse, entropy, kl f32 + is_clipped u8
    return 8 + 4 + 5 * 4 + 1


def per_row_bytes_bwd():
    # ids, old_logp, logp, lse, dloss in; zero_row out
    return 8 + 4 + 4 + 4 + 4 + 1


def copy_probe(torch):
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def cpu_baseline(case, old):
    """The float64 oracle on the whole workload (one step), timed on the host."""
    import oracle
    R = case.N
    reps = 0
    t0 = time.perf_counter()
    while True:   # whole steps until about 10 s of CPU work (at most 30 steps)
        z = oracle.decode_bf16(case.logits)
        fwd = oracle.grpo_forward(z, case.ids, old.astype(np.float64), None, case.adv,
                                  case.mask, case.B, case.L, case.temperature, case.beta,
                                  case.eps_low, case.eps_high)
        dz, g, zr = oracle.grpo_backward(z, case.ids, old.astype(np.float64), None, case.adv,
                                         case.mask, case.dloss, case.B, case.L,
                                         case.temperature, case.beta, case.eps_low,
                                         case.eps_high, fwd=fwd)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 30:
            break
    dt = (time.perf_counter() - t0) / reps
    nz = int((~zr).sum())
    nbytes = (R * case.V * 2 + R * per_row_bytes_fwd()
              + R * case.V * 2 + nz * case.V * 2 + R * per_row_bytes_bwd())
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full steps (fwd+bwd, {R} rows x {case.V} each) in float64 "
                      f"NumPy, {dt:.3f} s per step, single thread; {R / dt:.0f} rows/s; "
                      f"host CPU {cpu}"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the row pass shards by sequence with no exchange; see DESIGN.md).",
              file=sys.stderr)
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

    case = synth.grpo_token_case(with_ref=False, dloss="mean")
    logp_true = synth.load_stored_logp("token", case.logits[synth.stored_check_rows("token")])
    old = synth.add_noise_f32(logp_true, case.old_noise)
    B, L, V, N = case.B, case.L, case.V, case.N

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    z0 = torch.from_numpy(case.logits.view(np.int16)).view(torch.bfloat16).cuda()
    ids, old_t, adv, mask, dloss = dev(case.ids), dev(old), dev(case.adv), dev(case.mask), dev(case.dloss)
    sets = []
    for k in range(args.sets):
        z = z0.clone() if k else z0
        out = {n: torch.empty(N, dtype=torch.float32, device="cuda")
               for n in ("loss", "logp", "lse", "entropy", "kl")}
        out["is_clipped"] = torch.empty(N, dtype=torch.uint8, device="cuda")
        sets.append(dict(z=z, out=out, dz=torch.empty((N, V), dtype=torch.bfloat16, device="cuda"),
                         zr=torch.empty(N, dtype=torch.uint8, device="cuda")))
    kw = dict(temperature=case.temperature, beta=case.beta, eps_low=case.eps_low,
              eps_high=case.eps_high, level="token")

    # arguments are marshalled once per buffer set; a step is two C calls
    for s in sets:
        s["fwd"], _ = grl.grpo_logits_fwd(s["z"], ids, old_t, adv, B, L, mask=mask,
                                          out=s["out"], prepare=True, **kw)
        s["bwd"], _, _ = grl.grpo_logits_bwd(s["z"], ids, old_t, adv, B, L, s["out"]["logp"],
                                             s["out"]["lse"], dloss, mask=mask, dlogits=s["dz"],
                                             zero_row=s["zr"], prepare=True, **kw)

    def step(s, ev=None):
        if ev is not None:
            ev[0].record()
        s["fwd"]()
        if ev is not None:
            ev[1].record()
        s["bwd"]()
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    n_zero = int(sets[0]["zr"].sum().item())
    n_nz = N - n_zero

    # wall time of K steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # per-kernel durations over a second timed pass, events on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    fwd_bytes = N * V * 2 + N * per_row_bytes_fwd()
    bwd_bytes = N * V * 2 + n_nz * V * 2 + N * per_row_bytes_bwd()
    step_bytes = fwd_bytes + bwd_bytes
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    fwd_gbs = fwd_bytes / (fwd_ms * 1e-3) / 1e9
    bwd_gbs = bwd_bytes / (bwd_ms * 1e-3) / 1e9
    dom = ("grpo_bwd", bwd_gbs, bwd_ms, bwd_bytes) if bwd_ms >= fwd_ms else \
          ("grpo_fwd", fwd_gbs, fwd_ms, fwd_bytes)

    res = {
        "metric": "GRPO logits fwd+bwd GB/s & % HBM peak at B4 L512 V32000 bf16; rows/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "token-level GRPO logits fwd+bwd, B=4 L=512 V=32000 bf16 "
                        "(T=0.9, beta=0.04, eps 0.2/0.28, 2 of 4 advantages 0, ref = policy, "
                        "token-mean dloss, lengths U{256..512})",
            "rows": N, "V": V, "zero_rows": n_zero, "nonzero_rows": n_nz,
            "buffer_sets": args.sets, "accumulate": "fp32",
        },
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "rows_per_s": round(N / (ms_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "kernels": {
            "grpo_fwd": {"ms": round(fwd_ms, 5), "bytes": fwd_bytes, "GB/s": round(fwd_gbs, 1)},
            "grpo_bwd": {"ms": round(bwd_ms, 5), "bytes": bwd_bytes, "GB/s": round(bwd_gbs, 1)},
        },
        "roofline": {"kernel": dom[0], "bound": "hbm", "achieved": round(dom[1], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom[1] / HBM_PEAK_GBS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, old)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
