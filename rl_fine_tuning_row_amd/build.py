"""Build the HIP library libgrpo_rows.so in-tree for gfx950.

    python -m rl_fine_tuning_row_amd.build [-v]

Every source under csrc/ is compiled by hipcc into one shared library next
to this file.  Packed fp32 VALU instructions are switched off for device code
(``-packed-fp32-ops``); hipcc's host pass warns that it does not know that
feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgrpo_rows.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# the sources the row kernels are built from (every other file is the GEMM
# and the fused-linear path, which also uses the row kernels)
ROW_SOURCES = ("rows.hip", "row_core.hpp", "rows_internal.hpp", "host_common.hpp")


def source_digest(part: str = "all") -> str:
    """sha256 over the HIP sources, their headers and the C header (identifies
    the kernels a measurement was taken on).  part="rows" covers only the row
    kernels' sources (and the C header); "all" covers every source."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                   if f.endswith((".hip", ".hpp", ".h"))
                   and (part == "all" or f in ROW_SOURCES))
    files.append(os.path.join(INCLUDE, "grpo_rows.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        cmd = [hipcc, *COMMON, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in (r.stderr or "").splitlines()
                         if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
        return obj

    srcs = sources()
    with ThreadPoolExecutor(max(1, min(8, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    build_c_check(hipcc, verbose)
    return LIB_PATH


C_CHECK_SRC = os.path.join(ROOT, "tests", "c", "abi_check.cpp")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c", "abi_check")


def build_c_check(hipcc: str, verbose: bool = False) -> None:
    """Compile tests/c/abi_check.cpp, a C++ program that uses the library
    through the C ABI alone (linked against libgrpo_rows.so, found through a
    relative rpath)."""
    if not os.path.exists(C_CHECK_SRC):
        return
    cmd = [hipcc, *COMMON, "-I", INCLUDE, C_CHECK_SRC, "-L", PKG, "-lgrpo_rows",
           "-Wl,-rpath,$ORIGIN/../../rl_fine_tuning_row_amd", "-o", C_CHECK_BIN]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed on {C_CHECK_SRC}:\n{errs}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
