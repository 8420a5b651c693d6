#!/usr/bin/env python3
"""RMSNorm forward + backward benchmark on one MI355X.

A step is one pass of the whole path over one batch: the forward
(y, rstd), then the backward row kernel (dx and dW partials) and the
fixed-order dW combine, all through the C ABI on one HIP stream.

Measurement, following the Quack Hopper study ("What a tuned RMSNorm kernel
actually costs on Hopper", section 02):
  * the roofline denominator is measured in the same run: the best of a
    copy, a pure write and a two-read-one-write probe over 2 GiB buffers,
    probed again at the end (each pass after a short untimed load that
    brings the clocks up); the closing/opening ratio flags a drifting
    (shared) device, and the larger of the two passes is the denominator;
  * inputs rotate through R cloned sets that together exceed the last-level
    caches, and the backward of step k uses a different set than its
    forward, so no kernel reads data an earlier kernel just left in cache;
  * outputs are validated against the fp64 oracle before and after timing;
  * bytes are the algorithmic bytes the operation must touch (read x, w;
    write y, rstd for the forward; read x, dy, w, rstd and write dx, dW for
    the backward), never the dW partial traffic the kernels add.
Per-kernel times come from HIP events recorded around each launch inside the
timed region. A second, isolated measurement times single calls with a
1 GiB cache-flushing read before each (median of 50).

`python bench.py` prints one JSON line. `--gpus N` with N > 1 exits: this
build runs on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RMSNorm fwd/bwd achieved GB/s and % of measured HBM roofline, 1 MI355X"
HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
GIB = 1 << 30
SETTLE_S = 0.25  # untimed steps before the warmup steps (clock settle after the CPU leg)
PROBE_SETTLE_S = 0.3  # untimed copies before each roofline probe pass (clock settle)
PROBE_REPS = 25  # timed calls per probe variant and grid (median): with 11 the write probe's best moved ~1% between passes
CELL_SETTLE_S = 0.05  # untimed graph replays before each cell's timed replays
# Per-kernel graph length: launches per HIP graph, sized from the kernel's
# bytes so that one replay lasts about GRAPH_TARGET_MS (at least
# GRAPH_MIN_LAUNCHES launches), whatever --steps is. Short graphs made the
# average launch slower than the kernel's steady state (20 launches: 69.0 us
# against 65.0 us for the backward row kernel at bf16 16384 x 4096).
GRAPH_MIN_LAUNCHES, GRAPH_MAX_LAUNCHES, GRAPH_TARGET_MS = 200, 4000, 50.0
GRAPH_EST_GBPS = 6000.0   # for sizing only: a launch is estimated at its bytes / this rate, at least 5 us
SMALL_CELL_BYTES = 4 << 20  # cells with less than this per rotation set are timed call by call after a flush
CELL_ROTATION_BYTES = 2 * GIB  # larger cells rotate through at least this many bytes of sets
CELL_PARITY_ROWS = 64       # rows of y and dx each cell compares with the oracle (every rstd and dW column too)


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="bf16_16384x4096")
    ap.add_argument("--sets", type=int, default=0, help="rotation sets (0: enough to exceed 1.5 GiB, at least 4)")
    ap.add_argument("--probe-gib", type=float, default=2.0)
    ap.add_argument("--isolated-reps", type=int, default=50)
    ap.add_argument("--cpu-budget-s", type=float, default=20.0, help="time budget of the CPU-baseline leg")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle (profiling runs)")
    ap.add_argument("--eager-only", action="store_true",
                    help="per-kernel times from eager batches only, no HIP graphs (counter-collection runs)")
    ap.add_argument("--cells", default="all", help="cells mode: comma-separated groups (configs, formats, "
                    "residual, latency, element, pages) or all")
    ap.add_argument("--mode", default="bench", choices=["bench", "kernels", "copy", "cells"],
                    help="bench: full run; kernels: the warmup steps, then each kernel's graph replays "
                         "(eager batches with --eager-only), for profilers; "
                         "copy: one probe copy of --probe-gib (counter calibration)")
    ap.add_argument("--out-dir", default=os.environ.get("RMSN_BENCH_OUT", os.path.join(ROOT, "bench_out")))
    return ap.parse_args(argv)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


HOST_SOURCES = ("rmsn_api.cpp",)  # host code only: the ladder and the launches, no kernel


def source_hash() -> str:
    """Hash of the kernel sources (every file of csrc/ but the host-only
    HOST_SOURCES). Counter-derived traffic is reused only for this exact
    kernel code and, separately checked, the same launch configuration."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "memory_bound_normalization_rmsnorm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name in HOST_SOURCES:
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def launch_key(cfg: dict) -> list:
    """The fields of a launch configuration that decide a kernel's traffic: a
    trailing 1 for the LDS-staged backward (copy_mode 1), or the two-pass
    forward's vectors per lane kept in registers."""
    return [int(cfg[k]) for k in ("vector_path", "lanes_per_row", "vecs_per_lane", "wg_threads", "prefetch",
                                  "stream_loads", "grid")] + ([1] if cfg.get("copy_mode") else []) + \
        ([int(cfg["kept_vecs"])] if cfg.get("kept_vecs") else [])


def row_kernel_name(cfg: dict) -> str:
    """The backward row kernel a launch configuration runs (its template's name)."""
    vp = int(cfg["vector_path"])
    if vp == 0:
        return "bwd_scalar"
    if vp == 3:
        return "bwd_elem"
    if vp == 4:
        return "bwd_split"
    if vp == 2:
        return "bwd_wide_lds" if cfg.get("copy_mode") else "bwd_wide"
    return "bwd_lds" if cfg.get("copy_mode") else "bwd_vec"


def graph_launches(nbytes: int) -> int:
    """Launches per timing graph for a kernel moving `nbytes` per launch."""
    est_us = max(5.0, nbytes / (GRAPH_EST_GBPS * 1e3))
    return int(min(GRAPH_MAX_LAUNCHES, max(GRAPH_MIN_LAUNCHES, -(-GRAPH_TARGET_MS * 1e3 // est_us))))


def oracle_threads() -> int:
    """Threads of the all-cores oracle leg: the CPUs this process may run on,
    capped by OMP_NUM_THREADS when that is set (the host's share for this GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def git_rev() -> str:
    try:
        return subprocess.run(["git", "-C", ROOT, "rev-parse", "--short", "HEAD"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except Exception:
        return "unknown"


def _find(obj, key):
    """First value stored under `key` anywhere in a parsed JSON document."""
    if isinstance(obj, dict):
        if key in obj:
            return obj[key]
        obj = list(obj.values())
    if isinstance(obj, list):
        for v in obj:
            r = _find(v, key)
            if r is not None:
                return r
    return None


def smi_snapshot() -> dict:
    """GPU utilisation / VRAM as reported by the management tool (the run
    records it; a busy device makes every ratio suspect): graphics and memory
    controller activity (%) and VRAM in use, plus the tool's raw output."""
    for cmd in (["amd-smi", "metric", "--usage", "--mem-usage", "--json"],
                ["rocm-smi", "--showuse", "--showmemuse", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
            if r.returncode == 0 and r.stdout.strip():
                out = {"tool": cmd[0], "raw": r.stdout.strip()}
                try:
                    doc = json.loads(r.stdout)
                    for key in ("gfx_activity", "umc_activity", "used_vram", "total_vram"):
                        v = _find(doc, key)
                        out[key] = v.get("value") if isinstance(v, dict) else v
                except ValueError:
                    pass
                return out
        except Exception:
            continue
    return {"tool": None, "raw": "unavailable"}


def smi_brief(snap) -> dict | None:
    return None if snap is None else {k: snap.get(k) for k in ("tool", "gfx_activity", "umc_activity", "used_vram",
                                                                 "total_vram")}


def cpu_info() -> dict:
    model = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except Exception:
        avail = os.cpu_count()
    return {"model": model, "logical_cpus_available": avail}


class Timer:
    """HIP events on the current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def median_ms(self, fn, reps, warmup=3, between=None):
        torch = self.torch
        for _ in range(warmup):
            fn()
        times = []
        for _ in range(reps):
            if between is not None:
                between()
            s, e = self.event(), self.event()
            s.record()
            fn()
            e.record()
            e.synchronize()
            times.append(s.elapsed_time(e))
        torch.cuda.synchronize()
        return statistics.median(times), times


def probe_buffers(torch, gib):
    """The three probe buffers of `gib` GiB each (two inputs filled, one output)."""
    nbytes = int(gib * GIB) // 256 * 256
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    c = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b.fill_(2)
    return a, b, c


def probe_roofline(torch, rn, timer, gib, settle_s=PROBE_SETTLE_S, bufs=None):
    """Best of copy, pure write and 2-read-1-write over several grid sizes and
    cache hints (non-temporal loads and/or stores) (GB/s). A pure-read probe is
    reported beside them. Copies run untimed for settle_s of wall time first:
    a device that has just been idle (start-up, the CPU leg) needs tens of
    milliseconds of load before its clocks reach the level the timed kernels
    run at. `bufs` (from probe_buffers) lets two passes probe the same memory:
    the same probe on another 2 GiB allocation can differ by 1-2% with where
    the buffers land, which a drift check must not mistake for the device."""
    own = bufs is None
    a, b, c = probe_buffers(torch, gib) if own else bufs
    nbytes = a.numel()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < settle_s:
        for _ in range(8):
            rn.rmsn_probe_copy(a, c, nbytes, 0, 0)
        torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grids = [0, cus * 4, cus * 8, cus * 16, cus * 32]
    probes = {
        "copy": (lambda g, v: rn.rmsn_probe_copy(a, c, nbytes, g, v), 2 * nbytes),
        "write": (lambda g, v: rn.rmsn_probe_write(c, nbytes, g, v), nbytes),
        "2r1w": (lambda g, v: rn.rmsn_probe_add(a, b, c, nbytes, g, v), 3 * nbytes),
    }
    variants = {"copy": (0, 1, 2, 3), "write": (0, 2), "2r1w": (0, 1, 2, 3)}
    out = {}
    for name, (fn, moved) in probes.items():
        best = None
        for v in variants[name]:
            for g in grids:
                med, _ = timer.median_ms(lambda: fn(g, v), reps=PROBE_REPS, warmup=2)
                gbps = moved / (med * 1e-3) / 1e9
                if best is None or gbps > best[0]:
                    best = (gbps, g, v, med)
        out[name] = {"GBps": round(best[0], 1), "grid": best[1], "nt_variant": best[2], "median_ms": round(best[3], 4)}
    # a pure read, reported for information (the roofline is the best of the three above)
    sink = torch.zeros(64, dtype=torch.uint8, device="cuda")
    best = None
    for v in (0, 1):
        for g in grids:
            med, _ = timer.median_ms(lambda: rn.rmsn_probe_read(a, nbytes, sink, g, v), reps=PROBE_REPS, warmup=2)
            gbps = nbytes / (med * 1e-3) / 1e9
            if best is None or gbps > best[0]:
                best = (gbps, g, v, med)
    read = {"GBps": round(best[0], 1), "grid": best[1], "nt_variant": best[2], "median_ms": round(best[3], 4)}
    del a, b, c
    if own:
        torch.cuda.empty_cache()
    best_name = max(out, key=lambda k: out[k]["GBps"])
    return {"best_GBps": out[best_name]["GBps"], "best_probe": best_name, "probes": out, "read_GBps": read,
            "buffer_GiB": gib}


def size_matched_probes(torch, rn, nbytes, gib_total=1.5):
    """Copy and 2-read-1-write probes on tensors of the workload's own size
    (nbytes each), graph-timed, with inputs and outputs in separate rotating
    sets (so no call reads what a recent call wrote and the 256 MB MALL holds
    nothing useful). A short kernel pays its launch, ramp-up and drain on
    fewer bytes than a 2 GiB probe, so this is the ceiling a kernel of this
    size can reach. Best over non-temporal load/store variants, one 16-byte
    vector per lane."""
    R = max(3, -(-int(gib_total * GIB) // nbytes))
    ins = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2 * R)]
    outs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
    K = max(8, min(40, (4 * GIB) // nbytes))

    def graph_us(fn):
        for k in range(3):
            fn(k)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(K):
                fn(k)
        best = None
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            t = a.elapsed_time(b) * 1e3 / K
            best = t if best is None else min(best, t)
        del g
        return best

    out = {"tensor_bytes": nbytes, "rotation_sets": R}
    for name, moved, mk in (
            ("copy", 2 * nbytes, lambda v: lambda k: rn.rmsn_probe_copy(ins[k % R], outs[k % R], nbytes, 0, v)),
            ("2r1w", 3 * nbytes, lambda v: lambda k: rn.rmsn_probe_add(ins[k % R], ins[R + k % R], outs[k % R],
                                                                        nbytes, 0, v))):
        out[name + "_GBps"] = round(max(moved / graph_us(mk(v)) / 1e3 for v in (0, 1, 2, 3)), 1)
    del ins, outs
    torch.cuda.empty_cache()
    return out


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: the benchmark runs on one GPU only; "
                                   "RMSNorm rows shard across GPUs with no communication except one "
                                   "exchange of the N dW partial sums per GPU, which is not run here"}))
        return 2
    import numpy as np
    import torch

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs an MI355X (no GPU visible)")
    import memory_bound_normalization_rmsnorm_amd as rn
    import synthetic_inputs as si

    torch.cuda.set_device(0)
    timer = Timer(torch)
    props = torch.cuda.get_device_properties(0)

    if args.mode == "copy":
        nbytes = int(args.probe_gib * GIB) // 256 * 256
        a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        c = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        rn.rmsn_probe_copy(a, c, nbytes, 0)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read": nbytes, "bytes_written": nbytes}))
        return 0

    if args.mode == "cells":
        return run_cells(args, torch, rn, timer)

    wl = si.workload(args.workload)
    dt = rn.F32 if wl.dtype == "f32" else rn.BF16
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    M, N = wl.M, wl.N
    eps = si.eps_f32(wl.eps)
    fwd_bytes, bwd_bytes = wl.fwd_bytes(), wl.bwd_bytes()
    es = 4 if wl.dtype == "f32" else 2
    rows_bytes = 3 * M * N * es + N * es + 4 * M          # backward row kernel: x, dy, w, rstd in; dx out
    combine_bytes = 4 * N                                  # algorithmic part of the combine: dW out

    env = {
        "device": props.name, "gcn_arch": getattr(props, "gcnArchName", "?"),
        "compute_units": props.multi_processor_count, "hbm_GiB": round(props.total_memory / GIB, 1),
        "torch": torch.__version__, "hip": torch.version.hip, "library": rn.LIB_PATH,
        "build_info": rn.rmsnorm_build_info(), "git": git_rev(), "source_hash": source_hash(),
        "cpu": cpu_info(), "workload": wl.description,
        # the management tool is a script that re-execs its interpreter: only in full runs,
        # never under a profiler whose preload has already initialised the GPU
        "smi_at_start": smi_snapshot() if args.mode == "bench" else None,
    }
    log(f"device {props.name} ({props.multi_processor_count} CUs), library {rn.LIB_PATH}")

    do_full = args.mode == "bench"
    # the opening and closing passes probe the same buffers, held for the run
    probe_bufs = probe_buffers(torch, args.probe_gib) if do_full else None
    opening = probe_roofline(torch, rn, timer, args.probe_gib, bufs=probe_bufs) if do_full else None
    if opening:
        log(f"opening roofline {opening['best_GBps']} GB/s ({opening['best_probe']})")

    # ---- inputs -------------------------------------------------------------
    t0 = time.time()
    x_h, w_h, dy_h = si.make_inputs(wl)
    log(f"inputs generated in {time.time() - t0:.1f}s")

    def dev(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if wl.dtype == "bf16" else torch.from_numpy(a)
        return t.to("cuda")

    set_bytes = 4 * M * N * es + 4 * M
    R = args.sets or max(4, -(-int(1.5 * GIB) // set_bytes))
    w_d = dev(w_h)
    x0, dy0 = dev(x_h), dev(dy_h)
    sets = []
    for k in range(R):
        sets.append({
            "x": x0 if k == 0 else x0.clone(), "dy": dy0 if k == 0 else dy0.clone(),
            "y": torch.empty((M, N), dtype=tdt, device="cuda"), "dx": torch.empty((M, N), dtype=tdt, device="cuda"),
            "rstd": torch.empty(M, dtype=torch.float32, device="cuda"),
        })
    ws_bytes = rn.rmsnorm_bwd_workspace_bytes(M, N, dt)
    ldp_floats = -(-N // 64) * 64  # partial-row stride of the workspace
    ws = torch.empty(max(ws_bytes, 256) // 4, dtype=torch.float32, device="cuda")
    dw = torch.empty(N, dtype=torch.float32, device="cuda")
    cfg_f = rn.rmsnorm_query_config(M, N, dt, 0).as_dict()
    cfg_b = rn.rmsnorm_query_config(M, N, dt, 1).as_dict()
    log(f"{R} rotation sets; fwd config {cfg_f}; bwd config {cfg_b}")

    def fwd(s):
        rn.rmsnorm_fwd(s["x"], w_d, eps, M, N, dt, s["y"], s["rstd"])

    def bwd_rows(s):
        return rn.rmsnorm_bwd_rows(s["x"], w_d, s["dy"], s["rstd"], M, N, dt, s["dx"], ws, ws_bytes)

    def combine(p):
        rn.rmsnorm_bwd_combine(ws, p, N, dw)

    # rstd of every set (the backward reads the forward's rstd)
    for s in sets:
        fwd(s)
    torch.cuda.synchronize()

    validation = {}
    cpu_baseline = None

    def to_host(t):
        t = t.cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if wl.dtype == "bf16" else t.numpy()

    def snapshot():
        s = sets[0]
        fwd(s)
        combine(bwd_rows(s))
        torch.cuda.synchronize()
        return to_host(s["y"]), s["rstd"].cpu().numpy(), to_host(s["dx"]), dw.cpu().numpy()

    if do_full and not args.no_cpu_baseline:
        before = snapshot()
        cpu_baseline, oracle_ref = cpu_baseline_leg(wl, x_h, w_h, dy_h, eps, args.cpu_budget_s)
        validation["before_timing"] = validate(wl, before, oracle_ref, (x_h, w_h, dy_h))
        log(f"validation before timing: {validation['before_timing']}")

    # ---- timed steps ----------------------------------------------------------
    # K whole steps back to back (the JSON value), then, in the same warm
    # state, each kernel's average launch duration: K launches of it with the
    # same rotation captured in a HIP graph and replayed between one HIP event
    # pair on the launch stream (replay time / K). Graph replay removes the
    # host's launch rate (~7 us per launch from Python), which otherwise
    # bounds any kernel shorter than that; every replay's outputs are compared
    # bit for bit with the eager launches'. The eager batch (K launches
    # between one event pair) is reported beside it. (An event pair around
    # every single launch would add ~2 us of event processing per launch.)
    K, W = args.steps, args.warmup
    parts = [0] * R
    # --mode kernels launches only what the per-kernel figures time (the
    # warmup steps, then the graph replays; eager batches with --eager-only),
    # so a profiler's per-kernel averages cover the same launches
    kernels_only = args.mode == "kernels"

    def step(k):
        fwd(sets[k % R])
        combine(bwd_rows(sets[(k + R // 2) % R]))

    # Clock settle: the GPU idles while the CPU-baseline leg and validation
    # run (seconds), and its clocks take tens of milliseconds of load to come
    # back; 30 warmup steps (3.5 ms at the headline workload) left the first
    # part of the timed region slow (115.6 against 113.0 us per step after
    # 1000). So untimed steps run for SETTLE_S of wall time before the W
    # warmup steps, whatever W is: the timed region measures the loaded
    # steady state a training loop runs in.
    # idle check just before the timed region (the device should be ours alone)
    env["smi_before_timing"] = smi_snapshot() if args.mode == "bench" else None
    settle_steps, t_settle = 0, time.perf_counter()
    if not kernels_only:
        while time.perf_counter() - t_settle < SETTLE_S:
            for _ in range(32):
                step(settle_steps)
                settle_steps += 1
            torch.cuda.synchronize()
    for k in range(W):
        step(k)
    torch.cuda.synchronize()
    ms_per_step = step_event_ms = None
    if not kernels_only:
        e0, e1 = timer.event(), timer.event()
        t_start = time.perf_counter()
        e0.record()
        for k in range(K):
            step(k)
        e1.record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        step_event_ms = e0.elapsed_time(e1) / K
        ms_per_step = elapsed * 1e3 / K

    def batch(fn, n):
        a, b = timer.event(), timer.event()
        a.record()
        for k in range(n):
            fn(k)
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    def graph_batch(fn, outputs, KG, replays=3):
        """Per-launch us of KG launches of fn captured in a HIP graph: the median
        of `replays` timed replays after one untimed one. outputs(last) lists the
        tensors launch `last` writes (the last of the sequence); every replay's
        are checked against the eager launches' (the last R launches of the
        sequence, which write them)."""
        last = (KG - 1) % R
        for k in range(max(0, KG - R), KG):
            fn(k)
        torch.cuda.synchronize()
        ref = [t.clone() for t in outputs(last)]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(KG):
                fn(k)
        graph.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(replays):
            for t in outputs(last):
                t.fill_(float("nan"))
            torch.cuda.synchronize()
            a, b = timer.event(), timer.event()
            a.record()
            graph.replay()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / KG)
            for t, r in zip(outputs(last), ref):
                if not torch.equal(t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16),
                                   r.view(torch.int32) if r.dtype == torch.float32 else r.view(torch.int16)):
                    raise RuntimeError("graph replay output differs from the eager launches")
        del graph
        return statistics.median(times)

    def rows_k(k):
        parts[k % R] = bwd_rows(sets[(k + R // 2) % R])

    P_rows = cfg_b["partial_rows"]
    KG = {"fwd": graph_launches(fwd_bytes), "bwd_rows": graph_launches(rows_bytes),
          "combine": graph_launches(P_rows * ldp_floats * 4 + combine_bytes)}
    f_eager = r_eager = c_eager = None
    if args.eager_only or not kernels_only:
        # --eager-only (counter runs) launches K of each; otherwise as many as the graphs hold
        f_eager = batch(lambda k: fwd(sets[k % R]), K if args.eager_only else KG["fwd"])
        r_eager = batch(rows_k, K if args.eager_only else KG["bwd_rows"])
        c_eager = batch(lambda k: combine(parts[k % R]), K if args.eager_only else KG["combine"])
    if args.eager_only:
        f_us, r_us, c_us = f_eager, r_eager, c_eager
    else:
        f_us = graph_batch(lambda k: fwd(sets[k % R]), lambda last: (sets[last]["y"], sets[last]["rstd"]), KG["fwd"])
        r_us = graph_batch(rows_k, lambda last: (sets[(last + R // 2) % R]["dx"],
                                                 ws[:parts[last] * ldp_floats].view(parts[last], ldp_floats)[:, :N]),
                           KG["bwd_rows"])
        c_us = graph_batch(lambda k: combine(parts[k % R]), lambda last: (dw,), KG["combine"])
    def us(v):
        return "-" if v is None else f"{v:.1f}"

    if ms_per_step is not None:
        log(f"timed {K} steps: {ms_per_step * 1e3:.1f} us/step wall ({step_event_ms * 1e3:.1f} us by events)")
    log(f"per launch (graph / eager): fwd {us(f_us)} / {us(f_eager)} us, bwd rows {us(r_us)} / {us(r_eager)} us, "
        f"combine {us(c_us)} / {us(c_eager)} us")
    eager = None if f_eager is None else {"fwd_us": round(f_eager, 2), "bwd_rows_us": round(r_eager, 2),
                                          "combine_us": round(c_eager, 2)}

    if args.mode == "kernels":
        print(json.dumps({"mode": "kernels", "steps": K, "ms_per_step": ms_per_step, "fwd_us": f_us,
                          "bwd_rows_us": r_us, "combine_us": c_us, "eager": eager, "source_hash": env["source_hash"],
                          "graph_launches": None if args.eager_only else KG, "graph_replays": 3,
                          "fwd_launch": launch_key(cfg_f), "bwd_launch": launch_key(cfg_b)}))
        return 0

    # ---- isolated calls with a cache flush before each ------------------------
    # the flush reads 1 GiB (more than L2 + the 256 MB MALL) and writes nothing,
    # so no dirty lines are left to be written back during the timed call
    flush_n = GIB
    fa = torch.empty(flush_n, dtype=torch.uint8, device="cuda")
    fb = torch.zeros(64, dtype=torch.uint8, device="cuda")
    fa.fill_(3)
    torch.cuda.synchronize()

    def flush():
        rn.rmsn_probe_read(fa, flush_n, fb, 0)

    iso_f, iso_f_all = timer.median_ms(lambda: fwd(sets[0]), args.isolated_reps, between=flush)
    iso_b, iso_b_all = timer.median_ms(lambda: combine(bwd_rows(sets[0])), args.isolated_reps, between=flush)
    del fa, fb

    def spread(ms):
        # latency distribution of the isolated calls, us: min, p10, median, p90, max
        q = sorted(ms)
        at = lambda f: q[min(len(q) - 1, int(round(f * (len(q) - 1))))] * 1e3
        return {"min": round(q[0] * 1e3, 2), "p10": round(at(0.1), 2), "median": round(statistics.median(q) * 1e3, 2),
                "p90": round(at(0.9), 2), "max": round(q[-1] * 1e3, 2), "n": len(q)}

    if do_full and not args.no_cpu_baseline:
        validation["after_timing"] = validate(wl, snapshot(), oracle_ref, (x_h, w_h, dy_h))
        log(f"validation after timing: {validation['after_timing']}")

    sized = size_matched_probes(torch, rn, M * N * es)
    log(f"size-matched probes: {sized}")
    closing = probe_roofline(torch, rn, timer, args.probe_gib, bufs=probe_bufs)
    del probe_bufs
    drift = closing["best_GBps"] / opening["best_GBps"]
    # the denominator is the best the hardware showed in either pass, so a
    # slow opening pass cannot inflate the percentages
    measured = max(opening["best_GBps"], closing["best_GBps"])

    fwd_gbps = fwd_bytes / (f_us * 1e-6) / 1e9
    bwd_call_us = r_us + c_us
    bwd_gbps = bwd_bytes / (bwd_call_us * 1e-6) / 1e9
    rows_gbps = rows_bytes / (r_us * 1e-6) / 1e9
    value = (fwd_bytes + bwd_bytes) / (ms_per_step * 1e-3) / 1e9

    traffic = load_traffic(env["source_hash"], "bwd_rows", args.workload, launch_key(cfg_b))
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded PCG64 inputs on the host, uploaded once; rotated through cloned device buffers)",
        "config": {"workload": f"RMSNorm fwd+bwd {wl.dtype} M={M} N={N} eps={wl.eps}", "M": M, "N": N,
                   "eps": wl.eps, "rotation_sets": R, "fwd_launch": cfg_f, "bwd_launch": cfg_b},
        "roofline": {
            "kernel": f"{row_kernel_name(cfg_b)} (backward row kernel)",
            "bound": "hbm",
            "achieved": round(rows_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(rows_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": rows_bytes,
            "avg_launch_us": round(r_us, 2),
        },
        "measured_roofline": {"GBps": measured, "opening": opening, "closing_GBps": closing["best_GBps"],
                              "drift": round(drift, 4), "drift_ok": 0.99 <= drift <= 1.01,
                              "denominator": "the larger of the opening and closing passes' best probe"},
        "size_matched_roofline": dict(sized, fwd_pct_of_copy=round(100 * fwd_gbps / sized["copy_GBps"], 1),
                                      bwd_rows_pct_of_2r1w=round(100 * rows_gbps / sized["2r1w_GBps"], 1)),
        "fwd": {"avg_us": round(f_us, 2), "GBps": round(fwd_gbps, 1), "pct_measured_roofline": round(100 * fwd_gbps / measured, 1),
                "algorithmic_bytes": fwd_bytes, "isolated_median_us": round(iso_f * 1e3, 2),
                "isolated_GBps": round(fwd_bytes / (iso_f * 1e-3) / 1e9, 1), "isolated_us": spread(iso_f_all)},
        "bwd": {"avg_us": round(bwd_call_us, 2), "rows_kernel_us": round(r_us, 2), "combine_us": round(c_us, 2),
                "GBps": round(bwd_gbps, 1), "pct_measured_roofline": round(100 * bwd_gbps / measured, 1),
                "algorithmic_bytes": bwd_bytes, "isolated_median_us": round(iso_b * 1e3, 2),
                "isolated_GBps": round(bwd_bytes / (iso_b * 1e-3) / 1e9, 1), "isolated_us": spread(iso_b_all)},
        "step_event_us": round(step_event_ms * 1e3, 2),
        "settle_steps": settle_steps,
        "idle_check": {"at_start": smi_brief(env["smi_at_start"]),
                       "before_timing": smi_brief(env["smi_before_timing"])},
        "timing": "value: wall clock over K whole eager steps (synchronised at both ends), after untimed steps "
                  f"for {SETTLE_S} s (clock settle after the CPU leg) and W warmup steps; per-kernel avg_us: "
                  "graph_launches rotated launches of that kernel (about 50 ms of work, at least 200, whatever "
                  "K is) captured in a HIP graph, the median of 3 replays each between one HIP event pair on "
                  "the launch stream (outputs checked against eager); eager_batch_us: the same launches "
                  "issued eagerly between one event pair",
        "graph_launches": KG,
        "eager_batch_us": eager,
        "pct_measured_roofline": round(100 * value / measured, 1),
        "validation": validation,
        "cpu_baseline": cpu_baseline,
        "environment": {k: env[k] for k in ("device", "gcn_arch", "compute_units", "hip", "torch", "build_info",
                                             "git", "source_hash")},
    }
    os.makedirs(args.out_dir, exist_ok=True)
    env["smi_at_end"] = smi_snapshot()
    with open(os.path.join(args.out_dir, "environment.json"), "w") as f:
        json.dump(env, f, indent=1)
    with open(os.path.join(args.out_dir, "result.json"), "w") as f:
        json.dump(result, f, indent=1)
    print(json.dumps(result))
    return 0


# ---- the measurement cells ---------------------------------------------------
# Each cell is one shape and format, timed for one or more variants of the
# forward and the backward call:
#   fused     rmsnorm_fwd / rmsnorm_bwd (the library's path)
#   unfused   rmsn_unfused_fwd / rmsn_unfused_bwd (one kernel per step: the
#             row crosses HBM once per kernel)
#   residual  rmsnorm_fwd_residual / rmsnorm_bwd_residual (fused residual add)
#   residual_unfused  rmsn_add then rmsnorm_fwd; rmsnorm_bwd then rmsn_add
# GB/s is always the operation's algorithmic bytes over the call time, so a
# variant that moves more bytes shows up as a lower rate for the same work.
# Groups: the synthetic configurations; other storage formats ("What a tuned
# RMSNorm kernel actually costs on Hopper", section 07); the fused residual
# add ("Profiling, GPU utilisation and writing a fused kernel", Problem 15);
# the latency regime at d = 4096 (same page, the benchmark of Problem 15);
# rows that are not a multiple of 16 bytes (the element kernels);
# the shapes the other pages test (hello-gpu ch. 13 section 13.4 and 13.5;
# "RMSNorm backward (almost) without the column reduction", its benchmark).
CELL_GROUPS = {
    "configs": [("fp32_256x1024", "f32", 256, 1024), ("bf16_16384x4096", "bf16", 16384, 4096),
                ("bf16_32768x8192", "bf16", 32768, 8192), ("bf16_qknorm_1048576x128", "bf16", 1048576, 128),
                ("bf16_4096x32768", "bf16", 4096, 32768), ("bf16_16384x5120", "bf16", 16384, 5120),
                ("bf16_16384x7168", "bf16", 16384, 7168)],
    "formats": [("f16_16384x4096", "f16", 16384, 4096), ("bf16w32_16384x4096", "bf16w32", 16384, 4096),
                ("f16w32_16384x4096", "f16w32", 16384, 4096), ("bf16w32_32768x8192", "bf16w32", 32768, 8192),
                ("fp32_16384x4096", "f32", 16384, 4096), ("fp32_4096x32768", "f32", 4096, 32768)],
    "residual": [("bf16_16384x4096", "bf16", 16384, 4096), ("bf16_32768x8192", "bf16", 32768, 8192),
                 ("f16w32_16384x4096", "f16w32", 16384, 4096), ("bf16_1024x4096", "bf16", 1024, 4096)],
    "latency": [(f"bf16_{m}x4096", "bf16", m, 4096) for m in (1, 16, 256, 4096, 32768)],
    "element": [("bf16_16384x4100", "bf16", 16384, 4100), ("bf16_16384x4095", "bf16", 16384, 4095),
                ("fp32_16384x4098", "f32", 16384, 4098)],
    "pages": [("fp32_3x13", "f32", 3, 13), ("fp32_33x257", "f32", 33, 257), ("fp32_1024x4096", "f32", 1024, 4096),
              ("bf16_16384x8192", "bf16", 16384, 8192)],
}
CELL_VARIANTS = {"configs": ("fused", "unfused"), "formats": ("fused",), "residual": ("residual", "residual_unfused"),
                 "latency": ("fused", "unfused"), "element": ("fused",), "pages": ("fused", "unfused")}
FMT = {"f32": ("f32", 4, 4), "bf16": ("bf16", 2, 2), "f16": ("f16", 2, 2), "bf16w32": ("bf16", 2, 4),
       "f16w32": ("f16", 2, 4)}  # activation storage, activation bytes, weight bytes


def cell_bytes(variant, M, N, es, wsz):
    """Algorithmic bytes of one forward and one backward call of the operation."""
    if variant.startswith("residual"):
        # fwd: read x, res, w; write h, y, rstd. bwd: read h, dy, dh, w, rstd; write dx, dW
        return 4 * M * N * es + N * wsz + 4 * M, 4 * M * N * es + N * wsz + 4 * M + 4 * N
    return 2 * M * N * es + N * wsz + 4 * M, 3 * M * N * es + N * wsz + 4 * M + 4 * N


def run_cells(args, torch, rn, timer):
    """Time every cell's variants. Each variant is first checked against the
    fp64 oracle on the cell's own inputs (CELL_PARITY_ROWS rows of y and dx,
    every rstd, every dW column; the residual sum h bit for bit); a cell that
    fails gets no time. Cells of at least SMALL_CELL_BYTES per rotation set
    rotate through at least CELL_ROTATION_BYTES of sets and are timed as K
    calls captured in a HIP graph and replayed (the per-call time without
    host launch gaps), and as K eager launches between two events; every
    graph replay's outputs are compared with the eager call's, bit for bit.
    Smaller cells would sit in the 256 MB MALL however they rotate, so each
    of their calls is timed on its own between two events, after a 1 GiB
    cache-flushing read (the median of args.isolated_reps calls)."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity_util import to_host

    groups = list(CELL_GROUPS) if args.cells == "all" else args.cells.split(",")
    roof = probe_roofline(torch, rn, timer, args.probe_gib)
    measured = roof["best_GBps"]
    log(f"roofline {measured} GB/s ({roof['best_probe']})")
    codes = {"f32": rn.F32, "bf16": rn.BF16, "f16": rn.F16, "bf16w32": rn.BF16_WF32, "f16w32": rn.F16_WF32}
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    # the cache-flushing read of the small cells' isolated calls
    flush_a = torch.full((GIB,), 3, dtype=torch.uint8, device="cuda")
    flush_sink = torch.zeros(64, dtype=torch.uint8, device="cuda")

    def flush():
        rn.rmsn_probe_read(flush_a, GIB, flush_sink, 0)

    rows, failures = [], []
    sized = {}  # size-matched probes per tensor size
    for group in groups:
        for name, fmt, M, N in CELL_GROUPS[group]:
            act, es, wsz = FMT[fmt]
            code = codes[fmt]
            eps = float(np.float32(1e-6))
            gen = torch.Generator(device="cuda")
            gen.manual_seed(M * 7919 + N)
            variants = CELL_VARIANTS[group]
            resid = any(v.startswith("residual") for v in variants)
            per_set = M * N * es * (7 if resid else 4) + 4 * M
            small = per_set < SMALL_CELL_BYTES
            R = 2 if small else max(4, -(-CELL_ROTATION_BYTES // per_set))

            def randn(scale=1.0):
                return (torch.randn((M, N), generator=gen, device="cuda") * scale).to(tdt[act])

            base = {"x": randn(), "dy": randn(1e-2)}
            if resid:
                base["res"] = randn()
                base["dh"] = randn(1e-2)
            w = (1.0 + 0.1 * torch.randn(N, generator=gen, device="cuda")).to(torch.float32 if wsz == 4 else tdt[act])
            ref = cell_reference(base, w, eps, act, "f32" if wsz == 4 else act, M, N, to_host)
            sets = []
            for k in range(R):
                s = {key: (v if k == 0 else v.clone()) for key, v in base.items()}
                for key in ("y", "dx") + (("h",) if resid else ()):
                    s[key] = torch.empty((M, N), dtype=tdt[act], device="cuda")
                s["rstd"] = torch.empty(M, dtype=torch.float32, device="cuda")
                sets.append(s)
            ws_n = max(rn.rmsnorm_bwd_workspace_bytes(M, N, code),
                       rn.rmsn_unfused_bwd_workspace_bytes(M, N, code) if (N * es) % 16 == 0 else 0, 256)
            ws = torch.empty(ws_n // 4, dtype=torch.float32, device="cuda")
            dw = torch.empty(N, dtype=torch.float32, device="cuda")
            fb, bb = None, None
            for variant in variants:
                if variant.startswith("unfused") and (N * es) % 16 != 0:
                    continue  # the unfused kernels take the vector layout only
                fb, bb = cell_bytes(variant, M, N, es, wsz)
                ops = cell_ops(rn, variant, sets, w, dw, ws, ws_n, eps, M, N, code)
                rec = {"group": group, "cell": name, "format": fmt, "M": M, "N": N, "variant": variant,
                       "rotation_sets": R, "timing": "isolated" if small else "graph"}
                # every set's rstd (and h) for the backward; set 0's outputs checked against the oracle
                for k in range(R):
                    ops["fwd"](k)
                for t in ops["outputs_bwd"](0):
                    t.fill_(float("nan"))
                ops["bwd"](0)
                torch.cuda.synchronize()
                try:
                    rec["parity"] = cell_check(sets[0], dw, ref, act, variant, resid, to_host)
                except AssertionError as e:
                    rec["parity"] = {"passed": False, "error": str(e)[:500]}
                    failures.append(f"{name}/{variant}")
                    rows.append(rec)
                    log(json.dumps(rec))
                    continue
                for which, nbytes in (("fwd", fb), ("bwd", bb)):
                    if small:
                        med, times = timer.median_ms(lambda: ops[which](0), args.isolated_reps, between=flush)
                        best = med * 1e3
                        rec[which + "_isolated_us"] = round(best, 2)
                        rec[which + "_isolated_p10_p90_us"] = [round(sorted(times)[int(0.1 * (len(times) - 1))] * 1e3, 2),
                                                                round(sorted(times)[int(0.9 * (len(times) - 1))] * 1e3, 2)]
                        g_us, e_us = time_cell(torch, timer, ops[which], ops["outputs_" + which], R)
                        rec[which + "_warm_graph_us"] = round(g_us, 2)
                    else:
                        g_us, e_us = time_cell(torch, timer, ops[which], ops["outputs_" + which], R)
                        best = min(g_us, e_us)
                        rec[which + "_graph_us"] = round(g_us, 2)
                        rec[which + "_eager_us"] = round(e_us, 2)
                    rec[which + "_GBps"] = round(nbytes / (best * 1e-6) / 1e9, 1)
                    rec[which + "_pct_roofline"] = round(100 * nbytes / (best * 1e-6) / 1e9 / measured, 1)
                    rec[which + "_bytes"] = nbytes
                if not small:
                    # against streaming probes on tensors of the cell's own size: copy for the
                    # forward, 2-read-1-write for the backward
                    tb = M * N * es
                    if tb not in sized:
                        sized[tb] = size_matched_probes(torch, rn, tb)
                    rec["fwd_pct_size_matched"] = round(100 * rec["fwd_GBps"] / sized[tb]["copy_GBps"], 1)
                    rec["bwd_pct_size_matched"] = round(100 * rec["bwd_GBps"] / sized[tb]["2r1w_GBps"], 1)
                rows.append(rec)
                log(json.dumps(rec))
            del sets, base, ws, dw, ref
            torch.cuda.empty_cache()
    del flush_a, flush_sink
    out = {"mode": "cells", "roofline": roof, "cells": rows, "parity_failures": failures,
           "size_matched": {str(k): v for k, v in sized.items()},
           "timing": f"cells under {SMALL_CELL_BYTES >> 20} MiB per rotation set: the median of "
                     f"{args.isolated_reps} single calls, each between two HIP events after a 1 GiB "
                     "cache-flushing read (warm graph-replay times beside them); larger cells: rotation "
                     f"through at least {CELL_ROTATION_BYTES >> 30} GiB of input sets, the lower of the "
                     "graph-replay and eager per-call times"}
    os.makedirs(args.out_dir, exist_ok=True)
    with open(os.path.join(args.out_dir, "cells.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 1 if failures else 0


def cell_reference(base, w, eps, act, wdt, M, N, to_host):
    """The oracle's values for a cell, from host copies of its device inputs:
    y and dx on CELL_PARITY_ROWS rows spread over the cell (first and last
    included), r on every row and dW over every row (threads over row blocks,
    as the CPU-baseline leg), and the stored residual sum h on the sampled
    rows."""
    import numpy as np

    import oracle

    x = to_host(base["x"], act)
    dy = to_host(base["dy"], act)
    res = to_host(base["res"], act) if "res" in base else None
    dh = to_host(base["dh"], act) if "dh" in base else None
    wh = to_host(w, wdt)
    rows = np.unique(np.linspace(0, M - 1, min(M, CELL_PARITY_ROWS)).astype(np.int64))
    if res is None:
        oy, _ = oracle.fwd(x, wh, eps, act, rows=rows, wdtype=wdt)
        oh = None
    else:
        oh, oy, _ = oracle.fwd_residual(x, res, wh, eps, act, rows=rows, wdtype=wdt)
    odx, orr_rows = oracle.bwd_dx(x, wh, dy, eps, act, rows=rows, res=res, dh=dh, wdtype=wdt)
    _, r, _, dw = oracle_pass(x, wh, dy, eps, act, oracle_threads(), keep=False, wdtype=wdt, res=res, dh=dh,
                              rows_outputs=False)
    return {"rows": rows, "y": oy, "h": oh, "dx": odx, "r_rows": orr_rows, "rstd": r, "dw": dw,
            "x": x, "w": wh, "dy": dy, "dh": dh}


def cell_check(s, dw, ref, act, variant, resid, to_host):
    """Gates of one variant's outputs (rotation set 0) against the cell's
    oracle values; returns the statistics, raises AssertionError on a miss."""
    import numpy as np

    from parity_util import check_dw, check_rows, check_rstd, term_rms, widen

    rows = ref["rows"]
    out = {"rows_checked": int(rows.size)}
    y = to_host(s["y"], act)[rows]
    out["y_max_gate_ratio"] = check_rows(y, ref["y"], act, "y")["max_gate_ratio"]
    if resid:
        assert np.array_equal(widen(to_host(s["h"], act)[rows], act), ref["h"]), "stored residual sum h"
    extra = None
    if variant == "residual_unfused":
        # the normalisation's dx is rounded to storage before dh is added
        u = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}[act]
        extra = 2 * u * np.abs(ref["dx"] - widen(ref["dh"][rows], act))
    floor = term_rms(None, ref["w"], ref["dy"], ref["r_rows"], act, rows=rows, dh=ref["dh"])
    out["dx_max_gate_ratio"] = check_rows(to_host(s["dx"], act)[rows], ref["dx"], act, "dx", floor=floor,
                                          extra=extra)["max_gate_ratio"]
    out["rstd_max_rel_err"] = check_rstd(s["rstd"].cpu().numpy(), ref["rstd"])["max_rel_err"]
    d = check_dw(dw.cpu().numpy(), ref["dw"], act)
    out.update({"dw_max_rel_err": d["max_rel_err"], "dw_max_gate_ratio": d["max_gate_ratio"],
                "dw_cols_above_plain_rel_tol": d["cols_above_plain_rel_tol"], "passed": True})
    return out


def cell_ops(rn, variant, sets, w, dw, ws, ws_n, eps, M, N, code):
    """Forward and backward calls of a variant on rotation set k, and the
    outputs each writes (for the replay check)."""
    if variant == "fused":
        return {
            "fwd": lambda k: rn.rmsnorm_fwd(sets[k]["x"], w, eps, M, N, code, sets[k]["y"], sets[k]["rstd"]),
            "bwd": lambda k: rn.rmsnorm_bwd(sets[k]["x"], w, sets[k]["dy"], sets[k]["rstd"], M, N, code,
                                            sets[k]["dx"], dw, ws, ws_n),
            "outputs_fwd": lambda k: (sets[k]["y"], sets[k]["rstd"]), "outputs_bwd": lambda k: (sets[k]["dx"], dw)}
    if variant == "unfused":
        return {
            "fwd": lambda k: rn.rmsn_unfused_fwd(sets[k]["x"], w, eps, M, N, code, sets[k]["y"], sets[k]["rstd"]),
            "bwd": lambda k: rn.rmsn_unfused_bwd(sets[k]["x"], w, sets[k]["dy"], sets[k]["rstd"], M, N, code,
                                                 sets[k]["dx"], dw, ws, ws_n),
            "outputs_fwd": lambda k: (sets[k]["y"], sets[k]["rstd"]), "outputs_bwd": lambda k: (sets[k]["dx"], dw)}
    if variant == "residual":
        return {
            "fwd": lambda k: rn.rmsnorm_fwd_residual(sets[k]["x"], sets[k]["res"], w, eps, M, N, code, sets[k]["h"],
                                                     sets[k]["y"], sets[k]["rstd"]),
            "bwd": lambda k: rn.rmsnorm_bwd_residual(sets[k]["h"], w, sets[k]["dy"], sets[k]["dh"], sets[k]["rstd"],
                                                     M, N, code, sets[k]["dx"], dw, ws, ws_n),
            "outputs_fwd": lambda k: (sets[k]["h"], sets[k]["y"], sets[k]["rstd"]),
            "outputs_bwd": lambda k: (sets[k]["dx"], dw)}
    if variant == "residual_unfused":
        def fwd(k):
            s = sets[k]
            rn.rmsn_add(s["x"], s["res"], s["h"], M * N, code)
            rn.rmsnorm_fwd(s["h"], w, eps, M, N, code, s["y"], s["rstd"])

        def bwd(k):
            s = sets[k]
            rn.rmsnorm_bwd(s["h"], w, s["dy"], s["rstd"], M, N, code, s["dx"], dw, ws, ws_n)
            rn.rmsn_add(s["dx"], s["dh"], s["dx"], M * N, code)
        return {"fwd": fwd, "bwd": bwd, "outputs_fwd": lambda k: (sets[k]["h"], sets[k]["y"], sets[k]["rstd"]),
                "outputs_bwd": lambda k: (sets[k]["dx"], dw)}
    raise ValueError(variant)


def time_cell(torch, timer, op, outputs, R, replays=5):
    """(graph per-call us, eager per-call us) for op over the rotation sets.
    Two graph replays are checked first: every output is filled with NaN
    before each and must come back equal to the eager call's. Then replays run
    untimed for CELL_SETTLE_S (clock settle, as before the timed steps), then
    `replays` back to back between HIP events (the median per call), then the
    eager batch (K launches between one event pair)."""
    K = R * max(1, -(-16 // R))
    for k in range(K):
        op(k % R)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs((K - 1) % R)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(K):
            op(k % R)
    for _ in range(2):
        for t in outputs((K - 1) % R):
            t.fill_(float("nan"))  # a replay must rewrite every output
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs((K - 1) % R), ref):
            if not torch.equal(t.view(torch.uint8) if t.dtype != torch.float32 else t.view(torch.int32),
                               r.view(torch.uint8) if r.dtype != torch.float32 else r.view(torch.int32)):
                raise RuntimeError("graph replay output differs from the eager call")
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < CELL_SETTLE_S:
        graph.replay()
        torch.cuda.synchronize()
    ev = [timer.event() for _ in range(replays + 1)]
    ev[0].record()
    for i in range(replays):
        graph.replay()
        ev[i + 1].record()
    ev[-1].synchronize()
    times = [ev[i].elapsed_time(ev[i + 1]) * 1e3 / K for i in range(replays)]
    del graph
    e0, e1 = timer.event(), timer.event()
    e0.record()
    for k in range(K):
        op(k % R)
    e1.record()
    e1.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / K
    return statistics.median(times), eager_us


def load_traffic(src_hash, kernel, workload, launch):
    """HBM traffic per launch from committed rocprofv3 counter runs, only when
    they were taken on the current kernel sources and the same launch
    configuration; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(f"{kernel}:{workload}")
    if not entry or entry.get("source_hash") != src_hash or entry.get("launch") != launch:
        return None
    return entry.get("traffic_bytes_per_launch")


def oracle_pass(x, w, dy, eps, dtype, threads, keep=False, wdtype=None, res=None, dh=None, rows_outputs=True):
    """One whole pass of the fp64 oracle over a workload: forward (y, r) and
    backward dx for every row, and dW over every row (rows_outputs False: only
    r and dW; y and dx are not computed). The rows are split into
    `threads` contiguous blocks (a static schedule), one thread per block (the
    oracle's C code releases the GIL while it runs); each block's dW is summed
    over its own rows in fp64 and the block sums are added in block order, so
    the result does not depend on thread timing. Returns (y, r, dx, dw); y
    and dx only when `keep`, else None (each block's are dropped)."""
    import concurrent.futures

    import numpy as np

    import oracle

    M, N = x.shape
    T = max(1, min(int(threads), M)) if M else 1
    bounds = [(M * t // T, M * (t + 1) // T) for t in range(T)]
    y_all = np.empty((M, N)) if keep and rows_outputs else None
    dx_all = np.empty((M, N)) if keep and rows_outputs else None
    r_all = np.empty(M)

    def block(t):
        lo, hi = bounds[t]
        rows = np.arange(lo, hi, dtype=np.int64)
        sl = slice(lo, hi)
        if res is None:
            oy, orr = oracle.fwd(x, w, eps, dtype, rows=rows, wdtype=wdtype, want_y=rows_outputs)
        else:
            _, oy, orr = oracle.fwd_residual(x, res, w, eps, dtype, rows=rows, wdtype=wdtype, want_y=rows_outputs)
        if rows_outputs:
            odx, _ = oracle.bwd_dx(x, w, dy, eps, dtype, rows=rows, res=res, dh=dh, wdtype=wdtype)
        odw = oracle.bwd_dw(x[sl], dy[sl], eps, dtype, res=None if res is None else res[sl])
        r_all[sl] = orr
        if keep and rows_outputs:
            y_all[sl] = oy
            dx_all[sl] = odx
        return odw

    if T == 1:
        parts = [block(0)]
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=T) as ex:
            parts = list(ex.map(block, range(T)))
    dw = np.zeros(N)
    for p in parts:  # block order
        dw += p
    return y_all, r_all, dx_all, dw


def cpu_baseline_leg(wl, x, w, dy, eps, budget_s):
    """The fp64 oracle, as it stands, timed on this host over the whole
    workload (forward y and rstd, backward dx and dW, every row): single
    threaded, and on all the host CPUs this process may use (rows in static
    contiguous blocks, one per thread, per-thread dW added in thread order).
    Each variant is the median of up to 3 passes within `budget_s`. The last
    all-cores pass is kept as the validation reference. Returns (baseline
    record, reference)."""
    nbytes = wl.fwd_bytes() + wl.bwd_bytes()
    T = oracle_threads()

    def timed(threads, keep_last):
        times, out, t_start = [], None, time.perf_counter()
        for k in range(3):
            t0 = time.perf_counter()
            out = oracle_pass(x, w, dy, eps, wl.dtype, threads, keep=keep_last and k == 2)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget_s and k < 2:
                if keep_last:  # the reference needs the kept outputs
                    out = oracle_pass(x, w, dy, eps, wl.dtype, threads, keep=True)
                break
        return statistics.median(times), len(times), out

    t1, n1, _ = timed(1, False)
    tn, nn, ref = timed(T, True)
    info = cpu_info()
    record = {
        "value": round(nbytes / tn / 1e9, 4), "unit": "GB/s", "cores": T, "kind": "oracle",
        "sample": f"the whole workload ({wl.M} x {wl.N} {wl.dtype}): fp64 oracle forward (y, rstd) and backward "
                  f"(dx, dW) over every row, median of {nn} passes; rows split into {T} contiguous blocks, one "
                  "thread each, per-thread dW added in thread order; GB/s = the algorithmic bytes of one forward "
                  "and one backward call over the pass time",
        "seconds": round(tn, 3),
        "single_thread": {"value": round(nbytes / t1 / 1e9, 4), "unit": "GB/s", "cores": 1, "seconds": round(t1, 3),
                          "passes": n1},
        "cpu_model": info["model"], "logical_cpus_available": info["logical_cpus_available"],
    }
    log(f"cpu baseline: {record}")
    y, r, dx, dw = ref
    return record, {"y": y, "rstd": r, "dx": dx, "dw": dw}


def validate(wl, gpu, ref, inputs, block=2048):
    """Tolerance gates against the oracle on every row of y and dx (in blocks
    of rows), every rstd and every dW column. A failed gate raises: a wrong
    kernel gets no number."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity_util import check_dw, check_rows, check_rstd, term_rms

    x, w, dy = inputs
    y, rstd, dx, dw = gpu
    stats = {"y_max_abs_err": 0.0, "dx_max_abs_err": 0.0, "y_max_gate_ratio": 0.0, "dx_max_gate_ratio": 0.0}
    M = wl.M
    for lo in range(0, M, block):
        rows = slice(lo, min(M, lo + block))
        idx = list(range(rows.start, rows.stop))
        sy = check_rows(y[rows], ref["y"][rows], wl.dtype, "y")
        sdx = check_rows(dx[rows], ref["dx"][rows], wl.dtype, "dx",
                         floor=term_rms(x, w, dy, ref["rstd"][rows], wl.dtype, rows=idx))
        for k, st in (("y", sy), ("dx", sdx)):
            stats[k + "_max_abs_err"] = max(stats[k + "_max_abs_err"], st["max_abs_err"])
            stats[k + "_max_gate_ratio"] = max(stats[k + "_max_gate_ratio"], st["max_gate_ratio"])
    stats["rstd_max_rel_err"] = check_rstd(rstd, ref["rstd"])["max_rel_err"]
    dws = check_dw(dw, ref["dw"], wl.dtype)
    stats.update({"dw_max_rel_err": dws["max_rel_err"], "dw_max_gate_ratio": dws["max_gate_ratio"],
                  "dw_cols_above_plain_rel_tol": dws["cols_above_plain_rel_tol"], "dw_gate": dws["gate"]})
    stats["rows_checked"] = M
    stats["passed"] = True
    return stats


if __name__ == "__main__":
    sys.exit(main())
