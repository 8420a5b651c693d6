"""Build the C-ABI check program (tests/c_abi/rmsn_c_check): the library's
C entry points driven from C++ with no Python in the process, checked against
the fp64 oracle it links. Test infrastructure, built by the repository's
build step after the library."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "memory_bound_normalization_rmsnorm_amd")
BINARY = os.path.join(HERE, "rmsn_c_check")


def build(verbose: bool = False) -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    oracle_o = os.path.join(bdir, "rmsnorm_oracle.o")
    check_o = os.path.join(bdir, "rmsn_c_check.o")
    steps = [
        ["gcc", "-O2", "-std=c99", "-fPIC", "-c", os.path.join(ROOT, "oracle", "rmsnorm_oracle.c"), "-o", oracle_o],
        [hipcc, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-O2",
         "-std=c++17", "-c", os.path.join(HERE, "rmsn_c_check.cpp"), "-o", check_o],
        [hipcc, "--offload-arch=gfx950", check_o, oracle_o, "-L" + PKG, "-l:librmsnorm_mi355x.so",
         "-Wl,-rpath,$ORIGIN/../../memory_bound_normalization_rmsnorm_amd", "-o", BINARY + ".tmp"],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"C check build failed: {' '.join(cmd)}\n{res.stderr[-4000:]}")
        if verbose and res.stderr.strip():
            print(res.stderr[-2000:])
    os.replace(BINARY + ".tmp", BINARY)
    return BINARY


if __name__ == "__main__":
    print(build(verbose=True))
