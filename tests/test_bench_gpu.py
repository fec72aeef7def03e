"""bench.py's output line on the GPU: one JSON line with the contract's keys,
the roofline object and (GRPO workloads) the skip A/B and the with-reference
reading, for the headline and the tiny workload at a few steps (the other
workloads' "configs" object is left out here: it needs minutes of input
generation)."""
import json
import os
import subprocess
import sys

import pytest

from gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline")


@pytest.mark.parametrize("workload", ["grpo-token", "tiny"])
def test_bench_line(workload):
    require_gpu()
    say(f"bench line: {workload}")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload",
                        workload, "--steps", "5", "--warmup", "2", "--no-cpu-baseline",
                        "--no-configs"],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in KEYS:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2 and d["data"] == "synthetic"
    assert d["value"] > 0 and d["ms_per_step"] > 0 and "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma", "alu") and rf["peak"] > 0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    if workload == "grpo-token":
        assert d["higher_is_better"] is True and d["unit"] == "GB/s"
        ab = d["skip_ab"]
        assert ab["rounds"] == 5 and ab["skip_ms"] > 0 and ab["dense_ms"] > ab["skip_ms"]
        wr = d["with_reference"]
        assert wr["zero_rows"] < d["config"]["zero_rows"] and wr["single_pass"]["GB/s"] > 0
    else:
        assert d["higher_is_better"] is False and d["unit"] == "us"
