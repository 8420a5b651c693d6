"""The LDS-staged backward kernels (copy_mode 1: row blocks copied
global->LDS by direct-to-LDS loads into a ring of `prefetch` stages) against
the fp64 oracle, through the C ABI.

Every built (lanes per row, workgroup, stages) shape in every storage format,
plain and with the fused residual add, forced through
rmsnorm_{bwd,bwd_residual}_with_config:
  * a ragged row (the last wavefront partly past the row end),
  * a walk longer than the ring (each workgroup passes every stage more than
    once, ending on a partial row block),
  * a walk shorter than the ring (most of the prologue's copies are of rows
    past M),
and dW bit-identical when the call is repeated on fresh buffers.
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
from parity_util import check_dw, check_rows, check_rstd, gpu_bwd, gpu_fwd, gpu_fwd_residual, term_rms  # noqa: E402

# (lanes per row, workgroup, stages) built into the library (rmsn_instances.h)
LDS_SHAPES = [(256, 1024, 2), (256, 1024, 3), (256, 1024, 4), (512, 512, 2), (512, 512, 3), (512, 512, 4),
              (512, 512, 6), (512, 512, 8), (1024, 1024, 2), (1024, 1024, 3), (1024, 1024, 4), (0, 1024, 2),
              (0, 1024, 3), (0, 1024, 4)]
LDS_RES_SHAPES = [(256, 1024, 2), (256, 1024, 3), (512, 512, 2), (512, 512, 3), (512, 512, 4), (512, 512, 6),
                  (1024, 1024, 2), (1024, 1024, 3), (0, 1024, 2), (0, 1024, 3)]
FORMATS = ["f32", "bf16", "f16", "bf16w32", "f16w32"]
ROWWG_LANES = {2: 640, 3: 896, 4: 320}  # whole-wavefront rows exercised per stage count


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _shape_case(lpr, wg, st):
    """(lanes, nvec, rows per workgroup) of a ragged row for the shape."""
    if lpr == 0:
        lanes = ROWWG_LANES[st]
        return lanes, lanes - 37, 1
    return lpr, lpr // 2 + 3, wg // lpr


def _check(fmt, res, lpr, wg, st, M, grid, seed):
    act = "bf16" if fmt.startswith("bf16") else "f16" if fmt.startswith("f16") else "f32"
    wdt = "f32" if fmt.endswith("w32") or fmt == "f32" else act
    epv = 4 if act == "f32" else 8
    lanes, nvec, rpw = _shape_case(lpr, wg, st)
    N = nvec * epv
    x, w, dy = si.random_case(M, N, act, seed=seed, dy_scale=1e-2, w_dist="uniform", wdtype=wdt)
    eps = si.eps_f32(1e-6)
    cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=lanes, vecs_per_lane=1,
                            wg_threads=lanes if lpr == 0 else wg, prefetch=st, copy_mode=1, grid=grid)
    _say(f"lds {fmt} res={res} lanes={lanes} wg={wg} stages={st} M={M} N={N} grid={grid}")
    if res:
        r_in = si.random_tensor((M, N), act, seed=seed + 1)
        dh = si.random_tensor((M, N), act, seed=seed + 2, scale=1e-2)
        h, _, rstd = gpu_fwd_residual(x, r_in, w, eps, act)
        dx, dw = gpu_bwd(h, w, dy, rstd, act, cfg=cfg, dh=dh)
        odx, orr = oracle.bwd_dx(x, w, dy, eps, act, res=r_in, dh=dh, wdtype=wdt)
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
@pytest.mark.parametrize("fmt", FORMATS)
def test_every_lds_kernel(fmt, res):
    shapes = LDS_RES_SHAPES if res else LDS_SHAPES
    for lpr, wg, st in shapes:
        rpw = 1 if lpr == 0 else wg // lpr
        grid = 3
        # walk longer than the ring: each workgroup passes every stage twice and
        # ends on a partial row block
        M_long = (2 * st + 1) * grid * rpw + rpw // 2 + 1
        _check(fmt, res, lpr, wg, st, M_long, grid, seed=lpr * 7 + wg + st)
        # walk shorter than the ring: prologue copies of rows past M
        M_short = grid * rpw + 1
        _check(fmt, res, lpr, wg, st, M_short, grid, seed=lpr * 7 + wg + st + 1000)


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_lds_kernel_at_full_grid(fmt):
    """One LDS configuration per row shape at the workloads' own grid (one
    workgroup per compute unit) over 3000 rows (a ragged last pass), against
    the oracle on every row."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    epv = 4 if fmt == "f32" else 8
    # (vectors per row, lanes per row (0: the whole workgroup), workgroup, stages)
    for nvec, lpr, wg, st in ((512, 512, 512, 4), (256, 256, 1024, 3), (640, 0, 640, 3), (1024, 1024, 1024, 4)):
        N, M = nvec * epv, 3000
        x, w, dy = si.random_case(M, N, fmt, seed=N + st, dy_scale=1e-2)
        eps = si.eps_f32(1e-6)
        cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=nvec if lpr == 0 else lpr, vecs_per_lane=1,
                                wg_threads=wg, prefetch=st, copy_mode=1, grid=cus)
        _say(f"lds full grid {fmt} N={N} stages={st} grid={cus}")
        _, rstd = gpu_fwd(x, w, eps, fmt)
        dx, dw = gpu_bwd(x, w, dy, rstd, fmt, cfg=cfg)
        odx, orr = oracle.bwd_dx(x, w, dy, eps, fmt)
        check_rows(dx, odx, fmt, "dx", floor=term_rms(x, w, dy, orr, fmt))
        check_dw(dw, oracle.bwd_dw(x, dy, eps, fmt), fmt)


def test_lds_configuration_errors():
    """copy_mode 1 is refused for the forward, for shapes that are not built,
    and outside 2..8 stages."""
    M, N = 64, 4096
    x = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(N, dtype=torch.bfloat16, device="cuda")
    rstd = torch.ones(M, dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    dw = torch.empty(N, dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 22, dtype=torch.float32, device="cuda")
    bad = [dict(prefetch=1), dict(prefetch=9), dict(prefetch=5), dict(vecs_per_lane=2, lanes_per_row=256),
           dict(wg_threads=1024), dict(copy_mode=2)]
    for b in bad:
        c = dict(vector_path=1, lanes_per_row=512, vecs_per_lane=1, wg_threads=512, prefetch=4, copy_mode=1, grid=4)
        c.update(b)
        cfg = rn.rmsnorm_config(**c)
        with pytest.raises(rn.RmsnormError) as e:
            rn.rmsnorm_bwd_with_config(x, w, x, rstd, M, N, rn.BF16, out, dw, ws, ws.numel() * 4, cfg)
        assert e.value.status == rn.ECONFIG, b
    cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=128, vecs_per_lane=4, wg_threads=256, prefetch=2,
                            copy_mode=1, grid=4)
    with pytest.raises(rn.RmsnormError) as e:
        rn.rmsnorm_fwd_with_config(x, w, 1e-6, M, N, rn.BF16, out, rstd, cfg)
    assert e.value.status == rn.ECONFIG


# (lanes per row, vectors per lane, stages) of the wide-row LDS kernels (rmsn_instances.h)
WIDE_LDS_SHAPES = [(1024, 2, 1), (1024, 2, 2), (1024, 3, 1), (512, 4, 1), (512, 4, 2), (512, 6, 1)]


@pytest.mark.parametrize("fmt", ["bf16", "f16", "bf16w32", "f16w32"])
def test_every_wide_lds_kernel(fmt):
    """Wide rows (vector_path 2) with the next rows staged through LDS
    (copy_mode 1): every built shape, a ragged last vector slot, walks longer
    and shorter than the ring, against the oracle, and dW bit-identical on a
    second run."""
    act = "bf16" if fmt.startswith("bf16") else "f16"
    wdt = "f32" if fmt.endswith("w32") else act
    for lpr, vpt, st in WIDE_LDS_SHAPES:
        nvec = (vpt - 1) * lpr + lpr // 2 + 3
        N = nvec * 8
        grid = 3
        for M in ((2 * st + 1) * grid + 1, grid - 1):
            x, w, dy = si.random_case(M, N, act, seed=lpr + vpt * 7 + st + M, dy_scale=1e-2, w_dist="uniform",
                                      wdtype=wdt)
            eps = si.eps_f32(1e-5)
            cfg = rn.rmsnorm_config(vector_path=2, lanes_per_row=lpr, vecs_per_lane=vpt, wg_threads=lpr,
                                    prefetch=st, copy_mode=1, grid=grid)
            _say(f"wide lds {fmt} lanes={lpr} vpt={vpt} stages={st} M={M} N={N}")
            _, rstd = gpu_fwd(x, w, eps, act)
            dx, dw = gpu_bwd(x, w, dy, rstd, act, cfg=cfg)
            odx, orr = oracle.bwd_dx(x, w, dy, eps, act, wdtype=wdt)
            check_rows(dx, odx, act, "dx", floor=term_rms(x, w, dy, orr, act))
            check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act)
            dx2, dw2 = gpu_bwd(x, w, dy, rstd, act, cfg=cfg)
            assert np.array_equal(dw.view(np.uint32), dw2.view(np.uint32)), "dW differs between two runs"
