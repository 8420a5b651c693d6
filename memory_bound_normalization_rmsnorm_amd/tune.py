"""Launch-configuration search for the RMSNorm kernels, with an on-disk cache.

The library's default configuration comes from an analytical ladder on the
row width (``rmsnorm_select_config``). This module searches the space the
ladder chooses from -- lanes per row, workgroup size, grid, (forward)
non-temporal row loads, and the backward's memory path: register prefetch of
0-2 row blocks, or global->LDS copies into 2-8 LDS stages (copy_mode) -- by
timing each candidate through ``rmsnorm_{fwd,bwd}_with_config``.
It keeps the winner per (device, compute units, M, N, dtype, direction,
library build).

Scoring follows the benchmark's regime, not an L2-cold one: inputs rotate
through cloned buffer sets that together exceed the last-level caches, and
each candidate's K calls are captured in a HIP graph and replayed, so calls
shorter than the host's launch rate are timed by the device, not the host.
The Quack study ("What a tuned RMSNorm kernel actually costs on Hopper",
section 06) warns that a search scored in a different regime than the one
that runs regresses cells. The ladder's own choice is always a candidate, so
a tuned configuration is never slower than the default in the scoring regime,
up to timing noise. It also keeps the memory-path knobs (prefetch depth,
workgroup shape) in the search space, which that section asks for.

Note: the backward's dW bits depend on the configuration (the number of
partial rows sets the summation order). A tuned configuration is
deterministic run to run, but its dW bits differ from the default's.
"""

from __future__ import annotations

import json
import os
import statistics
import time

import torch

from . import (BF16, BF16_WF32, ECONFIG, F16, F16_WF32, F32, LIB_PATH, RmsnormError, lib, rmsnorm_bwd_with_config,
               rmsnorm_build_info, rmsnorm_config, rmsnorm_fwd_with_config, rmsnorm_query_config)

# activation element bytes, activation torch dtype and weight torch dtype of each format
ELEM = {F32: 4, BF16: 2, F16: 2, BF16_WF32: 2, F16_WF32: 2}
TORCH = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16, BF16_WF32: torch.bfloat16,
         F16_WF32: torch.float16}
WEIGHT = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16, BF16_WF32: torch.float32,
          F16_WF32: torch.float32}
# (lanes per row, workgroup sizes) built into the library; see csrc/rmsn_instances.h
BUILT = {1: (256,), 2: (256,), 4: (256,), 8: (256,), 16: (256,), 32: (256,), 64: (256, 512, 1024),
         128: (256, 512, 1024), 256: (256, 512, 1024), 512: (512, 1024), 1024: (1024,)}
MAX_VPT = 8
WIDE_LANES = 1024  # wide-row backward kernels (vector_path 2): 1024 lanes, dW sums in LDS
ELEM_LANES, ELEM_MAX = (64, 128, 256, 512, 1024), 16  # element kernels (vector_path 3): lanes, elements per lane
ROWWG_MIN_VECS = 256  # backward rows wider than this may run on any whole number of wavefronts
# LDS-staged backward kernels (copy_mode 1): (lanes per row, workgroup) -> stage counts built; lanes 0 is
# the row on the whole workgroup (see csrc/rmsn_instances.h)
LDS_BUILT = {(256, 1024): (2, 3, 4), (512, 512): (2, 3, 4, 6, 8), (1024, 1024): (2, 3, 4), (0, 1024): (2, 3, 4)}
# wide rows staged through LDS: (lanes per row, vectors per lane, stages)
WIDE_LDS_BUILT = ((1024, 2, 1), (1024, 2, 2), (1024, 3, 1), (512, 4, 1), (512, 4, 2), (512, 6, 1))
# vectors per lane of the plain forward's widest rows (1024 lanes)
FWD_XWIDE_VPT = 16
# the plain forward's two-pass kernels (vector_path 5): (chunk, vectors kept in
# registers between the passes, both in vectors per lane; copy_mode 1: the next
# 8 held in LDS)
_LOOP_16 = ((4, 0, 0), (8, 0, 0), (16, 0, 0), (4, 16, 0), (4, 12, 0), (2, 16, 1), (4, 16, 1), (4, 12, 1))
_LOOP_W32 = ((4, 0, 0), (8, 0, 0), (2, 14, 0), (2, 10, 1))
FWD_LOOP_BUILT = {BF16: _LOOP_16, F16: _LOOP_16,
                  F32: ((4, 0, 0), (8, 0, 0), (16, 0, 0), (2, 14, 0), (4, 12, 0), (2, 14, 1)),
                  BF16_WF32: _LOOP_W32, F16_WF32: _LOOP_W32}
# split-row backward kernels (vector_path 4): per format, vectors per lane -> prefetch variants
SPLIT_MAX = 16
SPLIT_BUILT = {
    BF16: {2: (0,), 3: (0, 1), 4: (0, 1)}, F16: {2: (0,), 3: (0, 1), 4: (0, 1)},
    BF16_WF32: {2: (0,), 3: (0,), 4: (0,)}, F16_WF32: {2: (0,), 3: (0,), 4: (0,)},
    F32: {5: (0,), 6: (0,), 7: (0,), 8: (0,)},
}
# split members that run two per CU (dW sums of at most 64 KiB): vectors per
# lane, 16-bit activations only
SPLIT_TWO_PER_CU = {BF16: 2, F16: 2, BF16_WF32: 2, F16_WF32: 2}
DEFAULT_CACHE = os.path.join(os.path.expanduser("~"), ".cache", "rmsnorm_mi355x", "tuned.json")


def cache_key(M: int, N: int, dtype: int, is_bwd: int, device_name: str, num_cus: int) -> str:
    build = rmsnorm_build_info()
    return f"{device_name}|{num_cus}|{build}|{'bwd' if is_bwd else 'fwd'}|{dtype}|{M}|{N}"


def candidates(M: int, N: int, dtype: int, is_bwd: int, num_cus: int, default: rmsnorm_config | None = None):
    """Every built vector shape that covers a row of N elements with one
    partially used slot at most, crossed with grids: the row-block count,
    its halves, and 1-4 workgroups per compute unit; for backward rows of more
    than 1024 vectors also the wide-row kernels at one and two workgroups per
    compute unit, for backward rows of 257 to 1024 vectors whose whole
    wavefronts are not a power of two the workgroup-sized row kernels, for
    forward rows of 8193 to 16384 vectors 9 to 16 vectors per lane on 1024
    lanes, for forward rows beyond 8192 vectors the two-pass kernels (every
    chunk size, a workgroup per row or two per CU), and for backward rows
    beyond the wide kernels the split-row kernels
    (the fewest members at one and at two per CU and one more of each,
    every built prefetch, resident groups and half of them). Shapes that are not built fail at launch and are skipped.
    Rows that are not a multiple of 16 bytes (up to 16384 columns) get the
    element kernels instead: the widest group of consecutive elements per
    access that N allows (pointers 16-byte aligned, as in the search's own
    buffers) and one element per access, on every row size from 64 to 1024
    lanes that holds the row in at most 16 elements per lane, each at the
    fewest accesses per lane, crossed with the row count, its half and 1, 2, 4
    and 8 workgroups per compute unit. Pure host logic."""
    es = ELEM[dtype]
    if (N * es) % 16:
        out = [default] if default is not None else []
        if N <= ELEM_LANES[-1] * ELEM_MAX:
            big = max(es, 4 if WEIGHT[dtype] == torch.float32 else 2)
            g = 1
            while 2 * g * big <= 16 and N % (2 * g) == 0:
                g *= 2
            grids = sorted(x for x in {M, -(-M // 2)} | {k * num_cus for k in (1, 2, 4, 8)} if 1 <= x <= M)
            for gg in sorted({g, 1}, reverse=True):
                for lanes in ELEM_LANES:
                    k = -(-N // (lanes * gg))
                    if k * gg > ELEM_MAX:
                        continue
                    for grid in grids:
                        out.append(rmsnorm_config(vector_path=3, lanes_per_row=lanes, vecs_per_lane=k,
                                                  elems_per_access=gg, wg_threads=lanes, grid=grid))
        return out
    nvec = N * es // 16
    out = []
    for lpr, wgs in BUILT.items():
        vpt = -(-nvec // lpr)
        if vpt > MAX_VPT:
            continue
        if vpt == 1 and lpr > 1 and nvec <= lpr // 2:
            continue  # half the lanes would hold the row as well
        if lpr < 64 and vpt > 1:
            continue  # narrow shapes are built with one vector per lane
        for wg in wgs:
            rpw = wg // lpr
            row_blocks = -(-M // rpw)
            grids = {row_blocks, -(-row_blocks // 2)} | {k * num_cus for k in (1, 2, 3, 4)}
            streams = (0, 1) if (not is_bwd and lpr >= 64) else (0,)
            depths = (0, 1, 2) if (is_bwd and vpt == 1) else (0, 1)  # depth 2: backward, one vector per lane
            for pf in depths:
                for g in sorted(x for x in grids if 1 <= x <= min(row_blocks, 1 << 20)):
                    for sl in streams:
                        out.append(rmsnorm_config(vector_path=1, lanes_per_row=lpr, vecs_per_lane=vpt,
                                                  wg_threads=wg, prefetch=pf, stream_loads=sl, grid=g))
    # backward rows of 257 to 1024 vectors on whole wavefronts (not a power of
    # two): the kernels whose row is the whole workgroup, one vector per lane
    rowwg = -(-nvec // 64) * 64
    if is_bwd and ROWWG_MIN_VECS < nvec <= WIDE_LANES and rowwg & (rowwg - 1):
        for pf in (1, 2):
            for g in sorted({k * num_cus for k in (1, 2, 3)} & set(range(1, M + 1))):
                out.append(rmsnorm_config(vector_path=1, lanes_per_row=rowwg, vecs_per_lane=1, wg_threads=rowwg,
                                          prefetch=pf, grid=g))
    # the LDS-staged backward: rows of one vector per lane, every built stage
    # count, one and two workgroups per compute unit
    if is_bwd and 256 <= nvec <= WIDE_LANES:
        lanes = 1 << (nvec - 1).bit_length()
        shapes = []
        if (lanes, 1024 if lanes == 256 else lanes) in LDS_BUILT and nvec > lanes // 2:
            shapes.append((lanes, 1024 if lanes == 256 else lanes, LDS_BUILT[(lanes, 1024 if lanes == 256 else lanes)]))
        if rowwg & (rowwg - 1):
            shapes.append((rowwg, rowwg, LDS_BUILT[(0, 1024)]))
        for lpr, wg, stages in shapes:
            rpw = wg // lpr
            row_blocks = -(-M // rpw)
            for st in stages:
                for g in sorted({k * num_cus for k in (1, 2)} & set(range(1, row_blocks + 1))) or [row_blocks]:
                    out.append(rmsnorm_config(vector_path=1, lanes_per_row=lpr, vecs_per_lane=1, wg_threads=wg,
                                              prefetch=st, copy_mode=1, grid=g))
    wide_max = 8 if dtype == F32 else 4
    if is_bwd and WIDE_LANES < nvec <= WIDE_LANES * wide_max:
        vpt = -(-nvec // WIDE_LANES)
        for pf in (0, 1):
            for g in sorted({num_cus, 2 * num_cus} & set(range(1, M + 1))):
                out.append(rmsnorm_config(vector_path=2, lanes_per_row=WIDE_LANES, vecs_per_lane=vpt,
                                          wg_threads=WIDE_LANES, prefetch=pf, grid=g))
        # the next rows staged through LDS (16-bit activations): one workgroup per CU
        if dtype != F32:
            for lpr, v, st in WIDE_LDS_BUILT:
                if (v - 1) * lpr < nvec <= v * lpr:
                    out.append(rmsnorm_config(vector_path=2, lanes_per_row=lpr, vecs_per_lane=v, wg_threads=lpr,
                                              prefetch=st, copy_mode=1, grid=min(num_cus, M)))
    # the plain forward's rows of 9 to 16 vectors per lane on 1024 lanes
    if not is_bwd and WIDE_LANES * MAX_VPT < nvec <= WIDE_LANES * FWD_XWIDE_VPT:
        vpt = -(-nvec // WIDE_LANES)
        for g in sorted(x for x in {M, num_cus, 2 * num_cus} if 1 <= x <= M):
            for sl in (0, 1):
                out.append(rmsnorm_config(vector_path=1, lanes_per_row=WIDE_LANES, vecs_per_lane=vpt,
                                          wg_threads=WIDE_LANES, stream_loads=sl, grid=g))
    # the forward's two-pass kernel, every built (chunk, kept, LDS) shape, for rows
    # beyond 8 vectors per lane (beyond 16 it is the only vector kernel)
    if not is_bwd and nvec > WIDE_LANES * MAX_VPT:
        for ch, kv, lds in FWD_LOOP_BUILT[dtype]:
            for g in sorted(x for x in {M, 2 * num_cus} if 1 <= x <= M):
                out.append(rmsnorm_config(vector_path=5, lanes_per_row=WIDE_LANES, vecs_per_lane=ch,
                                          wg_threads=WIDE_LANES, kept_vecs=kv, copy_mode=lds, grid=g))
    # backward rows beyond the wide kernels: split over K workgroups, the
    # fewest K whose slices fit at one and at two members per CU, and one
    # more of each, every built prefetch; groups of K as many as stay resident
    # and at most M, and half of them
    if is_bwd and nvec > WIDE_LANES * wide_max:
        ks = set()
        two = SPLIT_TWO_PER_CU.get(dtype, 0)
        for v in (wide_max, two) if two else (wide_max,):
            k0 = -(-nvec // (WIDE_LANES * v))
            ks |= {k0, k0 + 1}
        for K in sorted(ks):
            if K > SPLIT_MAX:
                continue
            slice_vecs = -(-nvec // K)  # vectors of each member's column slice
            vpt = -(-slice_vecs // WIDE_LANES)
            if vpt not in SPLIT_BUILT[dtype]:
                continue
            per_cu = 2 if vpt <= two else 1
            groups = min(per_cu * num_cus // K, M)
            for pf in SPLIT_BUILT[dtype][vpt]:
                for g in sorted({groups, -(-groups // 2)}):
                    if g >= 1:
                        out.append(rmsnorm_config(vector_path=4, lanes_per_row=K * WIDE_LANES, vecs_per_lane=vpt,
                                                  wg_threads=WIDE_LANES, prefetch=pf, grid=g * K))
    if default is not None:
        out.insert(0, default)
    return out


def _key(c: rmsnorm_config):
    return (c.vector_path, c.lanes_per_row, c.vecs_per_lane, c.wg_threads, c.prefetch, c.grid, c.stream_loads,
            c.elems_per_access, c.copy_mode, c.kept_vecs)


class _Bench:
    """Rotating device buffers for one (M, N, dtype) and a timer."""

    def __init__(self, M, N, dtype, sets_bytes=3 << 30, seed=0):
        self.M, self.N, self.dtype = M, N, dtype
        t = TORCH[dtype]
        per_set = 4 * M * N * ELEM[dtype] + 4 * M
        self.R = max(2, min(8, sets_bytes // max(per_set, 1)))
        g = torch.Generator(device="cuda").manual_seed(seed)
        self.sets = []
        for _ in range(self.R):
            self.sets.append(dict(
                x=torch.randn(M, N, device="cuda", generator=g).to(t),
                dy=(torch.randn(M, N, device="cuda", generator=g) * 1e-2).to(t),
                y=torch.empty(M, N, dtype=t, device="cuda"), dx=torch.empty(M, N, dtype=t, device="cuda"),
                rstd=torch.empty(M, device="cuda")))
        self.w = (1 + 0.1 * torch.randn(N, device="cuda", generator=g)).to(WEIGHT[dtype])
        self.dw = torch.empty(N, device="cuda")
        self.ws = None
        self.ws_bytes = 0

    def _ensure_ws(self, nbytes):
        if nbytes > self.ws_bytes:
            self.ws = torch.empty(nbytes // 4 + 64, device="cuda")
            self.ws_bytes = nbytes

    def run(self, cfg, is_bwd, k):
        s = self.sets[k % self.R]
        if is_bwd:
            rmsnorm_bwd_with_config(s["x"], self.w, s["dy"], s["rstd"], self.M, self.N, self.dtype, s["dx"], self.dw,
                                    self.ws, self.ws_bytes, cfg)
        else:
            rmsnorm_fwd_with_config(s["x"], self.w, 1e-6, self.M, self.N, self.dtype, s["y"], s["rstd"], cfg)

    def time_us(self, cfg, is_bwd, K=30, W=3, graph=True):
        """Per-call us of K rotated calls: captured in a HIP graph and replayed
        (the default; the host's launch rate would otherwise bound short
        calls), or issued eagerly between one event pair."""
        if is_bwd:
            ldp = -(-self.N // 64) * 64
            self._ensure_ws(int(cfg.grid) * ldp * 4)
        for k in range(W):
            self.run(cfg, is_bwd, k)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if not graph:
            a.record()
            for k in range(K):
                self.run(cfg, is_bwd, k)
            b.record()
            b.synchronize()
            return a.elapsed_time(b) * 1e3 / K
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(K):
                self.run(cfg, is_bwd, k)
        best = None
        for _ in range(3):
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            t = a.elapsed_time(b) * 1e3 / K
            best = t if best is None else min(best, t)
        del g
        return best


def tune(M: int, N: int, dtype: int, is_bwd: int, budget_s: float = 60.0, K: int = 30, verbose: bool = False,
         finalists: int = 4, rounds: int = 3):
    """Time the candidates (ladder default first) and return (best config, results).
    Stops early when the time budget is spent; the default is always timed.
    One timing per candidate ranks the sweep, but two configurations within a
    few percent of each other trade places from one timing to the next (at
    bf16 16384x4096 one sweep put a three-stage LDS ring 2.3% ahead of the
    ladder's two stages; five alternating timings each tied them within
    0.1%). So the `finalists` fastest and the default are timed again,
    `rounds` times each in alternation, and ranked by their median, which is
    what `results` then holds for them (the rest keep their one timing)."""
    if not torch.cuda.is_available():
        raise RuntimeError("tuning needs the GPU")
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    default = rmsnorm_query_config(M, N, dtype, is_bwd)
    bench = _Bench(M, N, dtype)
    fwd_default = rmsnorm_query_config(M, N, dtype, 0)
    for s in bench.sets:  # the backward reads the forward's rstd
        rmsnorm_fwd_with_config(s["x"], bench.w, 1e-6, M, N, dtype, s["y"], s["rstd"], fwd_default)
    torch.cuda.synchronize()
    t0 = time.time()
    results, seen = [], set()
    for cfg in candidates(M, N, dtype, is_bwd, props.multi_processor_count, default):
        if _key(cfg) in seen:
            continue
        seen.add(_key(cfg))
        if results and time.time() - t0 > budget_s:
            break
        try:
            us = bench.time_us(cfg, is_bwd, K=K)
        except RmsnormError as e:
            if e.status != ECONFIG:  # a HIP runtime error is not a shape that is not built
                raise
            continue
        results.append((us, cfg))
        if verbose:
            print(f"  {cfg.as_dict()} -> {us:.2f} us", flush=True)
    results.sort(key=lambda r: r[0])
    lead = [c for _, c in results[:finalists]]
    if _key(default) not in {_key(c) for c in lead}:
        lead += [c for _, c in results if _key(c) == _key(default)]
    times = {_key(c): [] for c in lead}
    for _ in range(rounds):
        for c in lead:
            times[_key(c)].append(bench.time_us(c, is_bwd, K=K))
    refined = sorted(((statistics.median(times[_key(c)]), c) for c in lead), key=lambda r: r[0])
    if verbose:
        for us, c in refined:
            print(f"  finalist {c.as_dict()} -> median {us:.2f} us", flush=True)
    done = {_key(c) for c in lead}
    results = refined + [r for r in results if _key(r[1]) not in done]
    return results[0][1], results


def best_config(M: int, N: int, dtype: int, is_bwd: int, cache_path: str = DEFAULT_CACHE, budget_s: float = 60.0,
                retune: bool = False) -> rmsnorm_config:
    """The cached winner for this shape on this device and library build; tunes
    (and stores) on a miss."""
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    key = cache_key(M, N, dtype, is_bwd, props.name, props.multi_processor_count)
    cache = load_cache(cache_path)
    if not retune and key in cache:
        return config_from_dict(cache[key]["config"])
    cfg, results = tune(M, N, dtype, is_bwd, budget_s=budget_s)
    default_us = next(us for us, c in results if _key(c) == _key(rmsnorm_query_config(M, N, dtype, is_bwd)))
    cache[key] = {"config": cfg.as_dict(), "us": results[0][0], "default_us": default_us,
                  "candidates_timed": len(results), "library": LIB_PATH}
    save_cache(cache_path, cache)
    return cfg


def config_from_dict(d: dict) -> rmsnorm_config:
    return rmsnorm_config(**{k: int(v) for k, v in d.items() if k in dict(rmsnorm_config._fields_)})


def load_cache(path: str) -> dict:
    try:
        with open(path) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def save_cache(path: str, cache: dict) -> None:
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(cache, f, indent=1, sort_keys=True)
    os.replace(tmp, path)


__all__ = ["best_config", "tune", "candidates", "cache_key", "config_from_dict", "load_cache", "save_cache", "lib"]
