"""Build of tests/c_abi_check.c (test infrastructure): the C ABI exercised
from plain C, linked against librba.so, the oracle's library and the HIP
runtime, with run paths relative to the binary so the tree can move."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_check.c")
BIN = os.path.join(HERE, "c_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = BIN):
    pkg = os.path.join(ROOT, "relative_position_bias_paged_amd")
    orc = os.path.join(ROOT, "oracle")
    rel_pkg = os.path.relpath(pkg, os.path.dirname(os.path.abspath(out)))
    rel_orc = os.path.relpath(orc, os.path.dirname(os.path.abspath(out)))
    return ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
            "-o", out, "-L", pkg, "-l:librba.so", "-L", orc, "-l:librba_oracle.so",
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
            f"-Wl,-rpath,$ORIGIN/{rel_pkg}", f"-Wl,-rpath,$ORIGIN/{rel_orc}",
            f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]


def build(out: str = BIN) -> str:
    res = subprocess.run(command(out), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("c_abi_check build failed:\n" + res.stderr[-4000:])
    return out
