"""Build the gfx950 RMSNorm library (``librmsnorm_mi355x.so``) in-tree with hipcc.

Each source compiles to an object in ``_build/`` (in parallel); the objects
link into a shared library next to this file, which the Python binding loads.
The measurement code (roofline probes, unfused reference kernels) links into
a second library, ``librmsnorm_mi355x_bench.so``, so the product carries none.
The kernel resource report (VGPRs, SGPRs, LDS, occupancy per kernel) that
hipcc prints is kept in ``_build/resource_usage.txt``.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "librmsnorm_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
BENCH_LIB_NAME = "librmsnorm_mi355x_bench.so"
BENCH_LIB_PATH = os.path.join(PKG, BENCH_LIB_NAME)

FORMATS = ["f32", "bf16", "f16", "bf16w32", "f16w32"]
SOURCES = ([f"rmsn_fwd_{f}.hip" for f in FORMATS] + [f"rmsn_bwd_{f}.hip" for f in FORMATS]
           + [f"rmsn_bwd_lds_{f}.hip" for f in FORMATS]
           + [f"rmsn_elem_l{lanes}.hip" for lanes in (64, 128, 256, 512, 1024)]
           + ["rmsn_common.hip", "rmsn_scratch.hip", "rmsn_api.cpp"])
BENCH_SOURCES = ["rmsn_probe.hip", "rmsn_baseline.hip"]
HEADERS = ["rmsn_device.h", "rmsn_tables.h", "rmsn_instances.h", "rmsn_fwd_kernels.h", "rmsn_fwd_loop.h",
           "rmsn_bwd_kernels.h", "rmsn_bwd_split.h",
           "rmsn_bwd_lds.h", "rmsn_elem_kernels.h"]
ARCH = "gfx950"
# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in generated code.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the gfx950 library cannot be built")
    return exe


def _git_rev() -> str:
    try:
        return subprocess.run(["git", "-C", PKG, "rev-parse", "--short", "HEAD"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except Exception:
        return "nogit"


def _compile(src: str, info: str, build_dir: str, extra: tuple) -> tuple[str, str]:
    path = os.path.join(CSRC, src)
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, f'-DRMSN_BUILD_INFO="{info}"', "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE_FLAGS + ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr[-6000:]}")
    return obj, res.stderr


def _link(objs, out: str, libs=()) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, *libs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed for {os.path.basename(out)}:\n{res.stderr[-4000:]}")
    os.replace(tmp, out)


def build(verbose: bool = False, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile every source for gfx950 and link the product library (and, in
    the tree, the measurement library beside it). Returns the product
    library's path. `out` and `extra_flags` (e.g. -D choices) build a variant
    of the product library elsewhere."""
    in_tree = out == LIB_PATH
    build_dir = BUILD if in_tree else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    extra = tuple(extra_flags)
    info = f"rmsnorm-mi355x {_git_rev()} {ARCH} hipcc -O3 -packed-fp32-ops {' '.join(extra)}".strip()
    sources = SOURCES + (BENCH_SOURCES if in_tree else [])
    workers = max(1, min(len(sources), os.cpu_count() or 4, 16))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda s: _compile(s, info, build_dir, extra), sources))
    objs = dict(zip(sources, (o for o, _ in results)))
    with open(os.path.join(build_dir, "resource_usage.txt"), "w") as f:
        for (o, log), s in zip(results, sources):
            f.write(f"==== {s}\n{log}\n")
    _link([objs[s] for s in SOURCES], out)
    if verbose:
        print(f"built {out}")
    if in_tree:
        # the unfused backward reuses the product's fixed-order dW combine
        _link([objs[s] for s in BENCH_SOURCES], BENCH_LIB_PATH,
              libs=("-L" + PKG, "-l:" + LIB_NAME, "-Wl,-rpath,$ORIGIN"))
        if verbose:
            print(f"built {BENCH_LIB_PATH}")
    return out


def is_stale() -> bool:
    """True when a library is missing or older than one of its sources."""
    inc = os.path.join(os.path.dirname(PKG), "include")
    incs = [os.path.join(inc, h) for h in os.listdir(inc)] if os.path.isdir(inc) else []
    for lib, srcs in ((LIB_PATH, SOURCES), (BENCH_LIB_PATH, BENCH_SOURCES)):
        if not os.path.exists(lib):
            return True
        t = os.path.getmtime(lib)
        deps = [os.path.join(CSRC, s) for s in srcs + HEADERS] + incs
        if any(os.path.getmtime(d) > t for d in deps if os.path.exists(d)):
            return True
    return False


if __name__ == "__main__":
    build(verbose=True)
