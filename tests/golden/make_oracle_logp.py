"""Write the oracle's float64 policy log-probabilities of the seeded workloads.

    python tests/golden/make_oracle_logp.py [token|sequence|tiny|fused ...]

The GRPO workloads form old_logp and ref_logp as the policy's own logp plus
noise.  That logp is the oracle's (float64, on the bf16-rounded logits; for
the fused workload on the logits h W^T of the bf16 hidden states and weight).
This script calls only ``oracle/`` and ``synth/`` and stores, per workload,
``oracle_logp_<name>.npy`` and ``oracle_lse_<name>.npy`` (float64 [B*L]) plus a digest of the bit patterns of a few
logits rows in ``oracle_logp_<name>.json`` so a loader can check that the
generators still produce the same inputs.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

CHECK_ROWS = (0, 1, 777)


def row_digest(rows: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(rows).tobytes()).hexdigest()


def blocked_logp(z_bits_or_none, get_block, n_rows, ids, T, block=128, threads=8):
    out = np.empty(n_rows, np.float64)
    lse = np.empty(n_rows, np.float64)

    def job(r0):
        r1 = min(n_rows, r0 + block)
        z = get_block(r0, r1)
        out[r0:r1], lse[r0:r1] = oracle.selective_log_softmax(z, ids[r0:r1], T)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(job, range(0, n_rows, block)))
    return out, lse


def make_grpo(case: synth.GrpoCase, name: str):
    t0 = time.time()
    z = case.logits

    def get_block(r0, r1):
        return oracle.decode_bf16(z[r0:r1])

    logp, lse = blocked_logp(None, get_block, case.N, case.ids, case.temperature)
    meta = {"name": name, "case": case.name, "rows": case.N, "V": case.V,
            "check_rows": list(CHECK_ROWS),
            "check_digest": row_digest(z[list(CHECK_ROWS)]),
            "note": "oracle float64 logp and lse of the bf16 logits at the workload's temperature"}
    return (logp, lse), meta, time.time() - t0


def make_tiny(case: synth.GrpoCase, name: str):
    """The tiny fp32 case (B=2 L=16 V=1024): check rows 0, 1 and the last."""
    t0 = time.time()
    z = case.logits
    logp, lse = oracle.selective_log_softmax(z.astype(np.float64), case.ids, case.temperature)
    rows = [0, 1, case.N - 1]
    meta = {"name": name, "case": case.name, "rows": case.N, "V": case.V,
            "check_rows": rows, "check_digest": row_digest(z[rows]),
            "note": "oracle float64 logp and lse of the fp32 logits at the workload's temperature"}
    return (logp, lse), meta, time.time() - t0


def make_fused(case: synth.FusedCase, name: str):
    t0 = time.time()
    h = oracle.decode_bf16(case.hidden)
    W = oracle.decode_bf16(case.weight)
    Wt = np.ascontiguousarray(W.T)

    def get_block(r0, r1):
        return h[r0:r1] @ Wt

    logp, lse = blocked_logp(None, get_block, case.N, case.ids, case.temperature, block=256,
                             threads=2)
    meta = {"name": name, "case": case.name, "rows": case.N, "V": case.V, "H": case.H,
            "check_rows": list(CHECK_ROWS),
            "check_digest": row_digest(case.hidden[list(CHECK_ROWS)]) + ":" +
            row_digest(case.weight[list(CHECK_ROWS)]),
            "note": "oracle float64 logp and lse of h W^T (bf16 h and W) at the workload's temperature"}
    return (logp, lse), meta, time.time() - t0


def save(name, logp_lse, meta):
    logp, lse = logp_lse
    np.save(os.path.join(HERE, f"oracle_logp_{name}.npy"), logp)
    np.save(os.path.join(HERE, f"oracle_lse_{name}.npy"), lse)
    with open(os.path.join(HERE, f"oracle_logp_{name}.json"), "w") as f:
        json.dump(meta, f, indent=1)


def main(which):
    if "token" in which:
        logp, meta, dt = make_grpo(synth.grpo_token_case(), "token")
        save("token", logp, meta)
        print(f"token: {dt:.1f}s")
    if "sequence" in which:
        logp, meta, dt = make_grpo(synth.grpo_sequence_case(), "sequence")
        save("sequence", logp, meta)
        print(f"sequence: {dt:.1f}s")
    if "tiny" in which:
        logp, meta, dt = make_tiny(synth.tiny_case("a"), "tiny")
        save("tiny", logp, meta)
        print(f"tiny: {dt:.1f}s")
    if "fused" in which:
        logp, meta, dt = make_fused(synth.fused_case(), "fused")
        save("fused", logp, meta)
        print(f"fused: {dt:.1f}s")


if __name__ == "__main__":
    main(sys.argv[1:] or ["token", "sequence", "tiny", "fused"])
