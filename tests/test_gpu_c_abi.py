"""The library through its C ABI alone: tests/c_abi/rmsn_c_check, a C++
program with no Python or torch in its process, runs the forward and the
backward on hipMalloc buffers for bf16 and fp32 shapes (vector, wide-row,
narrow-row, element and scalar kernels) and checks every output element against the
fp64 oracle it links. Built by the repository's build step."""

from __future__ import annotations

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

BINARY = os.path.join(os.path.dirname(__file__), "c_abi", "rmsn_c_check")


def test_c_abi_program_matches_oracle():
    assert os.path.exists(BINARY), f"{BINARY} is not built: run __graft_entry__.build()"
    res = subprocess.run([BINARY], capture_output=True, text=True, timeout=120)
    print(res.stdout[-3000:], flush=True)
    assert res.returncode == 0, f"rmsn_c_check failed ({res.returncode}):\n{res.stdout[-3000:]}\n{res.stderr[-2000:]}"
    assert res.stdout.strip().endswith("ok")


def test_host_time_per_call():
    """The host side of a decode-sized call, measured from C with no Python:
    argument checks, one lookup of the cached configuration and workspace
    size, and the launches. Printed for the record; bounded loosely here (a
    kernel of these shapes takes 2.5 to 5 us on the device)."""
    assert os.path.exists(BINARY), f"{BINARY} is not built: run __graft_entry__.build()"
    res = subprocess.run([BINARY, "--host-timing"], capture_output=True, text=True, timeout=120)
    print(res.stdout[-3000:], flush=True)
    assert res.returncode == 0, f"rmsn_c_check --host-timing failed:\n{res.stdout[-3000:]}\n{res.stderr[-2000:]}"
    import re
    times = [float(m) for m in re.findall(r"median ([0-9.]+) us", res.stdout)]
    assert len(times) == 7 and max(times) < 50.0, times
