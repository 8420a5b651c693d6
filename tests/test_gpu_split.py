"""Rows wider than one workgroup's share, against the fp64 oracle through
the C ABI:

  * the backward's split-row kernels (vector_path 4: each row on K
    workgroups of 1024 lanes that exchange their parts of the row sum through
    the workspace): every built (vectors per lane, prefetch) in every storage
    format, plain and residual-fused, forced by explicit configurations with
    ragged last slices, walks of several rows per group (both exchange values
    in use), groups without rows, and K from 2 to 16;
  * the plain forward's rows of 9 to 16 vectors per lane on 1024 lanes;
  * the forward's two-pass kernels (vector_path 5: rows beyond those, read
    in chunks, the first ones kept in registers, the next ones held in LDS,
    the rest read twice), every built (chunk, kept, LDS) shape, plain and
    residual-fused;
  * the ladder's own choice at 65536 and 131072 columns (bf16, fp16 with fp32
    weights, fp32, the residual-fused pair), every row and every dW column,
    and dW bit-identical on reruns.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import memory_bound_normalization_rmsnorm_amd as rn  # noqa: E402
import oracle  # noqa: E402
import synthetic_inputs as si  # noqa: E402
from parity_util import (check_dw, check_rows, check_rstd, gpu_bwd, gpu_fwd, gpu_fwd_residual,  # noqa: E402
                         oracle_row_blocks, term_rms, widen)

# (vectors per lane, prefetch) built per format (rmsn_instances.h)
SPLIT_SHAPES = {"bf16": [(2, 0), (3, 0), (3, 1), (4, 0), (4, 1)],
                "f16": [(2, 0), (3, 0), (3, 1), (4, 0), (4, 1)],
                "bf16w32": [(2, 0), (3, 0), (4, 0)], "f16w32": [(2, 0), (3, 0), (4, 0)],
                "f32": [(5, 0), (6, 0), (7, 0), (8, 0)]}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fmt(fmt):
    act = "bf16" if fmt.startswith("bf16") else "f16" if fmt.startswith("f16") else "f32"
    wdt = "f32" if fmt.endswith("w32") or fmt == "f32" else act
    return act, wdt, (4 if act == "f32" else 8)


def _split_nvec(K, vpt, short=None):
    """Vectors per row whose K slices hold (vpt - 1) * 1024 + 517 vectors each,
    the last one `short` fewer (K - 1 by default): ragged wavefronts in every
    slice and a shorter last slice."""
    sl = (vpt - 1) * 1024 + 517
    return K * sl - (K - 1 if short is None else short)


def _run_split(fmt, res, K, vpt, pf, M, groups, seed):
    act, wdt, epv = _fmt(fmt)
    N = _split_nvec(K, vpt) * epv
    x, w, dy = si.random_case(M, N, act, seed=seed, dy_scale=1e-2, w_dist="uniform", wdtype=wdt)
    eps = si.eps_f32(1e-6)
    cfg = rn.rmsnorm_config(vector_path=4, lanes_per_row=K * 1024, vecs_per_lane=vpt, wg_threads=1024, prefetch=pf,
                            grid=groups * K)
    _say(f"split {fmt} res={res} K={K} vpt={vpt} pf={pf} M={M} N={N} groups={groups}")
    if res:
        r_in = si.random_tensor((M, N), act, seed=seed + 1)
        dh = si.random_tensor((M, N), act, seed=seed + 2, scale=1e-2)
        h, _, rstd = gpu_fwd_residual(x, r_in, w, eps, act)
        dx, dw = gpu_bwd(h, w, dy, rstd, act, cfg=cfg, dh=dh)
        odx, orr = oracle.bwd_dx(x, w, dy, eps, act, res=r_in, dh=dh, wdtype=wdt)
        check_rstd(rstd, orr)
        check_rows(dx, odx, act, "dx", floor=term_rms(h, w, dy, orr, act, dh=dh))
        check_dw(dw, oracle.bwd_dw(x, dy, eps, act, res=r_in), act)
        dx2, dw2 = gpu_bwd(h, w, dy, rstd, act, cfg=cfg, dh=dh)
    else:
        _, rstd = gpu_fwd(x, w, eps, act)
        check_rstd(rstd, oracle.fwd(x, w, eps, act, want_y=False, wdtype=wdt)[1])
        dx, dw = gpu_bwd(x, w, dy, rstd, act, cfg=cfg)
        odx, orr = oracle.bwd_dx(x, w, dy, eps, act, wdtype=wdt)
        check_rows(dx, odx, act, "dx", floor=term_rms(x, w, dy, orr, act))
        check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act)
        dx2, dw2 = gpu_bwd(x, w, dy, rstd, act, cfg=cfg)
    assert np.array_equal(dw.view(np.uint32), dw2.view(np.uint32)), "dW differs between two runs"
    assert np.array_equal(dx.view(np.uint8), dx2.view(np.uint8)), "dx differs between two runs"


@pytest.mark.parametrize("res", [False, True], ids=["plain", "residual"])
@pytest.mark.parametrize("fmt", list(SPLIT_SHAPES))
def test_every_split_kernel(fmt, res):
    for vpt, pf in SPLIT_SHAPES[fmt]:
        # 3 groups over 8 rows: walks of 2 and 3 rows (both exchange values
        # in use, the prefetch past M on the last row)
        _run_split(fmt, res, 2, vpt, pf, 8, 3, seed=vpt * 10 + pf)


@pytest.mark.parametrize("fmt,K,vpt,pf,M,groups", [
    ("bf16", 3, 4, 1, 11, 4),     # odd K
    ("bf16", 5, 3, 1, 4, 2),
    ("f32", 3, 8, 0, 5, 2),
    ("bf16", 16, 3, 1, 3, 2),     # the widest split: 16 members
    ("bf16", 2, 4, 1, 2, 5),      # more groups than rows: three write zero partial rows
    ("f16w32", 4, 4, 0, 1, 1),    # one row, one group: dW straight from the group
])
def test_split_members_and_groups(fmt, K, vpt, pf, M, groups):
    _run_split(fmt, False, K, vpt, pf, M, groups, seed=K * 100 + M)


def test_split_configuration_errors():
    """Explicit split configurations that do not fit are refused before any
    launch: grid not whole groups, more workgroups than stay resident, K
    outside 2..16, slices wider than the kernel, shapes not built, forward."""
    M, N = 16, 65536
    x = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(N, dtype=torch.bfloat16, device="cuda")
    rstd = torch.ones(M, dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    dw = torch.empty(N, dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 24, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    base = dict(vector_path=4, lanes_per_row=2048, vecs_per_lane=4, wg_threads=1024, prefetch=1, grid=4)
    bad = [dict(grid=3), dict(grid=2 * cus + 2), dict(lanes_per_row=1024), dict(lanes_per_row=17 * 1024, grid=17),
           dict(lanes_per_row=1536), dict(vecs_per_lane=3), dict(vecs_per_lane=5), dict(prefetch=2),
           dict(copy_mode=1), dict(wg_threads=512)]
    for b in bad:
        c = dict(base)
        c.update(b)
        with pytest.raises(rn.RmsnormError) as e:
            rn.rmsnorm_bwd_with_config(x, w, x, rstd, M, N, rn.BF16, out, dw, ws, ws.numel() * 4,
                                       rn.rmsnorm_config(**c))
        assert e.value.status == rn.ECONFIG, b
    with pytest.raises(rn.RmsnormError) as e:
        rn.rmsnorm_fwd_with_config(x, w, 1e-6, M, N, rn.BF16, out, rstd, rn.rmsnorm_config(**base))
    assert e.value.status == rn.ECONFIG
    # a workspace one byte short of the exchange slots
    need = 2 * N * 4 + 256
    with pytest.raises(rn.RmsnormError) as e:
        rn.rmsnorm_bwd_with_config(x, w, x, rstd, M, N, rn.BF16, out, dw, ws, need - 1, rn.rmsnorm_config(**base))
    assert e.value.status == rn.EWORKSPACE


@pytest.mark.parametrize("fmt", ["bf16", "f16w32", "f32"])
def test_forward_rows_of_9_to_16_vectors_per_lane(fmt):
    """The plain forward on one 1024-lane workgroup per row, every vectors per
    lane from 9 to 16 (the last wavefront ragged), against the oracle."""
    act, wdt, epv = _fmt(fmt)
    for vpt in range(9, 17):
        N = ((vpt - 1) * 1024 + 517) * epv
        M = 5
        x, w, _ = si.random_case(M, N, act, seed=vpt, wdtype=wdt)
        eps = si.eps_f32(1e-6)
        cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=1024, vecs_per_lane=vpt, wg_threads=1024, grid=3)
        _say(f"forward {fmt} vpt={vpt} N={N}")
        y, rstd = gpu_fwd(x, w, eps, act, cfg=cfg)
        oy, orr = oracle.fwd(x, w, eps, act, wdtype=wdt)
        check_rows(y, oy, act, "y")
        check_rstd(rstd, orr)


# (chunk, kept, LDS-held) shapes (vectors per lane) of the two-pass forward
# kernels per format, plain and residual-fused (rmsn_instances.h); copy_mode 1
# holds 8 vectors per lane in LDS
_L16 = [(4, 0, 0), (8, 0, 0), (16, 0, 0), (4, 16, 0), (4, 12, 0), (2, 16, 8), (4, 16, 8), (4, 12, 8)]
_R16 = [(4, 0, 0), (8, 0, 0), (2, 16, 0), (4, 12, 0), (2, 16, 8), (4, 12, 8)]
_LW = [(4, 0, 0), (8, 0, 0), (2, 14, 0), (2, 10, 8)]
_RW = [(4, 0, 0), (8, 0, 0), (4, 8, 0), (4, 8, 8)]
LOOP_SHAPES = {"bf16": (_L16, _R16), "f16": (_L16, _R16),
               "f32": ([(4, 0, 0), (8, 0, 0), (16, 0, 0), (2, 14, 0), (4, 12, 0), (2, 14, 8)],
                       [(4, 0, 0), (8, 0, 0), (2, 12, 0), (4, 8, 0), (2, 12, 8)]),
               "bf16w32": (_LW, _RW), "f16w32": (_LW, _RW)}


def _loop_rows(ch, kv, lv):
    """Row lengths (vectors) for a two-pass shape: the kept and held chunks
    full, then two and a half reloaded chunks and a ragged wavefront; for
    shapes that keep vectors, a row that ends inside the kept part; for shapes
    that hold vectors in LDS, one that ends inside the held part."""
    rows = [(kv + lv) * 1024 + 2 * ch * 1024 + ch * 512 + 37]
    if kv:
        rows.append(kv * 1024 - ch * 512 - 37)
    if lv:
        rows.append(kv * 1024 + lv * 512 + 37)
    return rows


@pytest.mark.parametrize("res", [False, True], ids=["plain", "residual"])
@pytest.mark.parametrize("fmt", list(LOOP_SHAPES))
def test_every_forward_two_pass_kernel(fmt, res):
    """Every built (chunk, kept, LDS-held) shape, 5 rows on 3 workgroups (a
    workgroup takes a second row), on rows that reload chunks after the kept
    and held ones, rows that end inside the kept part and rows that end
    inside the held part: y and rstd against the oracle, and with the
    residual add h bit-exact."""
    act, wdt, epv = _fmt(fmt)
    for ch, kv, lv in LOOP_SHAPES[fmt][1 if res else 0]:
        for nvec in _loop_rows(ch, kv, lv):
            N, M = nvec * epv, 5
            x, w, _ = si.random_case(M, N, act, seed=ch + kv + lv + 31 * res, wdtype=wdt)
            eps = si.eps_f32(1e-6)
            cfg = rn.rmsnorm_config(vector_path=5, lanes_per_row=1024, vecs_per_lane=ch, wg_threads=1024,
                                    kept_vecs=kv, copy_mode=1 if lv else 0, grid=3)
            _say(f"two-pass forward {fmt} res={res} chunk={ch} kept={kv} lds={lv} N={N}")
            if res:
                r_in = si.random_tensor((M, N), act, seed=ch + kv + lv + 7)
                h, y, rstd = gpu_fwd_residual(x, r_in, w, eps, act, cfg=cfg)
                oh, oy, orr = oracle.fwd_residual(x, r_in, w, eps, act, wdtype=wdt)
                assert np.array_equal(widen(h, act), oh), "h differs from round(x + res)"
            else:
                y, rstd = gpu_fwd(x, w, eps, act, cfg=cfg)
                oy, orr = oracle.fwd(x, w, eps, act, wdtype=wdt)
            check_rows(y, oy, act, "y")
            check_rstd(rstd, orr)


# (format, M, N, residual): the ladder's own configuration
LADDER_CASES = [("bf16", 1024, 65536, False), ("bf16", 512, 131072, False), ("f16w32", 512, 131072, False),
                ("f32", 512, 65536, False), ("bf16", 512, 65536, True), ("bf16", 300, 131072 + 8, False),
                ("bf16", 1, 131072, False), ("bf16", 64, 262144, False), ("f32", 64, 131072, False),
                ("bf16", 64, 98304, True), ("bf16", 64, 131072 + 8, True), ("f32", 64, 65536, True),
                ("bf16", 64, 196608, False), ("f16w32", 64, 196608, False), ("bf16", 32, 262144, True),
                ("f32", 32, 98304, True)]


@pytest.mark.parametrize("fmt,M,N,res", LADDER_CASES, ids=lambda v: str(v))
def test_ladder_wide_rows_against_oracle(fmt, M, N, res):
    """Forward and backward at 65536 to 262144 columns as the library picks
    them (the backward on split rows; the forward on 1024 lanes holding 8 to
    16 vectors each, or beyond that the two-pass kernel): every row of y and
    dx, every rstd, every dW column; the backward twice, bit-identical."""
    act, wdt, _ = _fmt(fmt)
    x, w, dy = si.random_case(M, N, act, seed=N + M, dy_scale=1e-2, wdtype=wdt)
    eps = si.eps_f32(1e-6)
    code = {"bf16": rn.BF16, "f16w32": rn.F16_WF32, "f32": rn.F32}[fmt]
    q = rn.rmsnorm_query_config(M, N, code, 1).as_dict()
    _say(f"ladder {fmt} M={M} N={N} res={res}: backward {q}")
    assert q["vector_path"] == 4
    if res:
        r_in = si.random_tensor((M, N), act, seed=N + 1)
        dh = si.random_tensor((M, N), act, seed=N + 2, scale=1e-2)
        h, y, rstd = gpu_fwd_residual(x, r_in, w, eps, act)
        _, oy, orr = oracle.fwd_residual(x, r_in, w, eps, act, wdtype=wdt)
        check_rows(y, oy, act, "y")
        check_rstd(rstd, orr)
        dx, dw = gpu_bwd(h, w, dy, rstd, act, dh=dh)
        odx, _ = oracle.bwd_dx(x, w, dy, eps, act, res=r_in, dh=dh, wdtype=wdt)
        check_rows(dx, odx, act, "dx", floor=term_rms(h, w, dy, orr, act, dh=dh))
        check_dw(dw, oracle.bwd_dw(x, dy, eps, act, res=r_in), act)
        dx2, dw2 = gpu_bwd(h, w, dy, rstd, act, dh=dh)
    else:
        y, rstd = gpu_fwd(x, w, eps, act)
        dx, dw = gpu_bwd(x, w, dy, rstd, act)
        orr = np.empty(M)
        for rows, oy, r, odx in oracle_row_blocks(x, w, dy, eps, act, block=256, wdtype=wdt):
            orr[rows] = r
            check_rows(y[rows], oy, act, "y")
            idx = np.arange(rows.start, rows.stop)
            check_rows(dx[rows], odx, act, "dx", floor=term_rms(x, w, dy, r, act, rows=idx))
        check_rstd(rstd, orr)
        check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act)
        dx2, dw2 = gpu_bwd(x, w, dy, rstd, act)
    assert np.array_equal(dw.view(np.uint32), dw2.view(np.uint32)), "dW differs between two runs"
    assert np.array_equal(dx.view(np.uint8), dx2.view(np.uint8)), "dx differs between two runs"


@pytest.mark.parametrize("name", list(si.WIDE_WORKLOADS))
def test_full_size_wide_workload(name):
    """The wide-row workloads the benchmark can time (bf16 4096x65536: split
    rows over 4 workgroups, the forward at 8 vectors per lane; bf16
    1024x262144: 16 split-row members, the two-pass forward) at full size in
    the ladder's configuration: every row of y and dx against the oracle,
    every rstd, every dW column."""
    wl = si.WIDE_WORKLOADS[name]
    _say(f"wide workload {name}: generating inputs")
    x, w, dy = si.make_inputs(wl)
    eps = si.eps_f32(wl.eps)
    _say(f"wide workload {name}: gpu")
    y, rstd = gpu_fwd(x, w, eps, wl.dtype)
    dx, dw = gpu_bwd(x, w, dy, rstd, wl.dtype)
    _say(f"wide workload {name}: oracle, every row")
    orr = np.empty(wl.M)
    for rows, oy, r, odx in oracle_row_blocks(x, w, dy, eps, wl.dtype, block=128):
        orr[rows] = r
        check_rows(y[rows], oy, wl.dtype, "y")
        idx = np.arange(rows.start, rows.stop)
        check_rows(dx[rows], odx, wl.dtype, "dx", floor=term_rms(x, w, dy, r, wl.dtype, rows=idx))
    check_rstd(rstd, orr)
    check_dw(dw, oracle.bwd_dw(x, dy, eps, wl.dtype), wl.dtype)
    assert np.all(np.isfinite(widen(y, wl.dtype))) and np.all(np.isfinite(widen(dx, wl.dtype)))

