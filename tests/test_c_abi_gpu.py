"""The C ABI used from C++ alone: tests/c/abi_check (built by build() from
tests/c/abi_check.cpp) allocates with hipMalloc, calls the entry points of
include/grpo_rows.h and checks the invariants listed in its header."""
import os
import subprocess

import pytest

from gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_check")


def test_c_abi_program():
    require_gpu()
    assert os.path.exists(BIN), "tests/c/abi_check is not built (run __graft_entry__.build())"
    say("C ABI check program: fp32 3x40x1003 (T 0.9), bf16 3x40x4096, one fused-linear chunk")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-2000:]
    assert "abi_check ok" in r.stdout
