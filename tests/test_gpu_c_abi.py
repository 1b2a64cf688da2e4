"""The C ABI from plain C on the GPU: tests/c_abi_check (built by
__graft_entry__.build() from tests/c_abi_check.c) allocates with hipMalloc,
runs a decode and a prefill through librba.so over a shuffled page table and
compares every output element with the oracle's library, for a global and a
windowed layer, with no Python or torch in the process."""
import os
import subprocess

import pytest

from gpu_helpers import device

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_program_matches_the_oracle():
    device()
    assert os.path.exists(BIN), "tests/c_abi_check is missing: run __graft_entry__.build() first"
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("all ok")
    assert res.stdout.count(" ok") >= 4
