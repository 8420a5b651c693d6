"""GPU parity for the other storage formats and the fused residual add.

Formats: fp16 activations and weights, and fp32 (master) weights with bf16 or
fp16 activations ("What a tuned RMSNorm kernel actually costs on Hopper",
section 07: the weight format is a dimension of its own). Fused residual add
(page "Profiling, GPU utilisation and writing a fused kernel", Problem 15):
the stored sum h must equal the oracle's round(x + res) bit for bit, since both
sides round the exact sum once; y, rstd, dx and dW take the gates of the plain
path, with the residual gradient dh counted in dx's cancellation floor.
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
from parity_util import (FORMATS, check_dw, check_rows, check_rstd, gpu_bwd, gpu_fwd,  # noqa: E402
                         gpu_fwd_residual, term_rms, to_device, to_host, widen, workspace)

NEW_FORMATS = ("f16", "bf16w32", "f16w32")
ALL_FORMATS = tuple(FORMATS)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(M, N, fmt, seed, dy_scale=1e-2):
    act, wst, _ = FORMATS[fmt]
    x, w, dy = si.random_case(M, N, act, seed=seed, dy_scale=dy_scale, wdtype=wst)
    return act, wst, x, w, dy


def plain_check(x, w, dy, eps, act, wst, cfg=None):
    y, rstd = gpu_fwd(x, w, eps, act, cfg=cfg)
    oy, orr = oracle.fwd(x, w, eps, act, wdtype=wst)
    check_rows(y, oy, act, "y")
    check_rstd(rstd, orr)
    dx, dw = gpu_bwd(x, w, dy, rstd, act, cfg=cfg)
    odx, orr = oracle.bwd_dx(x, w, dy, eps, act, wdtype=wst)
    check_rows(dx, odx, act, "dx", floor=term_rms(x, w, dy, orr, act))
    check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act)


def residual_check(x, res, w, dy, dh, eps, act, wst, cfg=None, rows=None):
    """Fused residual forward and backward against the oracle's unfused
    composition. rows: compare only these rows of y and dx (full-size runs)."""
    h, y, rstd = gpu_fwd_residual(x, res, w, eps, act, cfg=cfg)
    oh, oy, orr = oracle.fwd_residual(x, res, w, eps, act, rows=rows, wdtype=wst)
    sel = slice(None) if rows is None else rows
    assert np.array_equal(widen(h[sel], act), oh), "h differs from round(x + res)"
    check_rows(y[sel], oy, act, "y (residual)")
    if rows is None:
        check_rstd(rstd, orr)
    else:
        check_rstd(rstd[rows], orr)
    dx, dw = gpu_bwd(h, w, dy, rstd, act, cfg=cfg, dh=dh)
    odx, orr = oracle.bwd_dx(x, w, dy, eps, act, rows=rows, res=res, dh=dh, wdtype=wst)
    hs = h if rows is None else h[rows]
    check_rows(dx[sel], odx, act, "dx (residual)",
               floor=term_rms(hs, w, dy, orr, act, rows=rows, dh=dh))
    check_dw(dw, oracle.bwd_dw(x, dy, eps, act, res=res), act, "dW (residual)")
    return h, y, rstd, dx, dw


SHAPES = [(1, 1), (3, 13), (33, 257), (7, 8), (17, 128), (129, 1000), (64, 1024), (31, 4096),
          (19, 5120), (9, 7168), (3, 8192), (2, 32768), (300, 96), (1000, 16)]


@pytest.mark.parametrize("fmt", NEW_FORMATS)
@pytest.mark.parametrize("M,N", SHAPES, ids=lambda v: str(v))
def test_formats_small(M, N, fmt):
    _say(f"formats_small M={M} N={N} {fmt}")
    act, wst, x, w, dy = _case(M, N, fmt, seed=2000 + M * 7 + N)
    plain_check(x, w, dy, si.eps_f32(1e-5), act, wst)


def _ladder_shapes():
    """The (lanes_per_row, vecs_per_lane, wg_threads, prefetch) kernels built for
    every format: the workgroups the ladder picks per width."""
    out = []
    for pf in (0, 1):
        out += [(lpr, 1, 256, pf) for lpr in (1, 2, 4, 8, 16, 32)]
        out += [(lpr, 1, 1024, pf) for lpr in (64, 128, 256)]
        for lpr in (64, 128, 256, 512, 1024):
            out += [(lpr, v, max(256, lpr), pf) for v in range(1, 9)]
    return out


def _ragged(lpr, vpt, wg, epv):
    nvec = min(lpr * vpt, max(1, lpr * (vpt - 1) + max(1, lpr // 2 + 1)))  # the last slot is partial
    return 3 * (wg // lpr) + 1, nvec * epv


@pytest.mark.parametrize("fmt", NEW_FORMATS)
def test_every_ladder_kernel(fmt):
    """Each kernel built for the format, forced through *_with_config on a ragged
    row, a ragged row count and a grid of 2 (workgroups loop over row blocks)."""
    shapes = _ladder_shapes()
    assert len(shapes) == 98
    for lpr, vpt, wg, pf in shapes:
        M, N = _ragged(lpr, vpt, wg, 8)
        cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=lpr, vecs_per_lane=vpt, wg_threads=wg,
                                prefetch=pf, grid=2)
        _say(f"kernel lpr={lpr} vpt={vpt} wg={wg} pf={pf} N={N} M={M} {fmt}")
        act, wst, x, w, dy = _case(M, N, fmt, seed=lpr * 100 + vpt + wg + pf)
        plain_check(x, w, dy, si.eps_f32(1e-6), act, wst, cfg=cfg)


@pytest.mark.parametrize("fmt", NEW_FORMATS)
def test_formats_scalar_and_unaligned(fmt):
    M, N = 37, 4096
    act, wst, x, w, dy = _case(M, N, fmt, seed=78)
    plain_check(x, w, dy, si.eps_f32(1e-5), act, wst, cfg=rn.rmsnorm_config(vector_path=0, grid=5))
    xd = to_device(np.concatenate([x.reshape(-1)[:1], x.reshape(-1)]))[1:]
    wd = to_device(np.concatenate([w[:1], w]))[1:]
    oy, orr = oracle.fwd(x, w, si.eps_f32(1e-5), act, wdtype=wst)
    for forced in (None, rn.rmsnorm_config(vector_path=0, grid=5)):   # the ladder (element kernels), the scalar
        y = torch.full((M * N + 1,), float("nan"), dtype=xd.dtype, device="cuda")[1:]
        rstd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        if forced is None:
            rn.rmsnorm_fwd(xd, wd, si.eps_f32(1e-5), M, N, FORMATS[fmt][2], y, rstd)
        else:
            rn.rmsnorm_fwd_with_config(xd, wd, si.eps_f32(1e-5), M, N, FORMATS[fmt][2], y, rstd, forced)
        torch.cuda.synchronize()
        check_rows(to_host(y, act).reshape(M, N), oy, act, "y (unaligned)")
        check_rstd(rstd.cpu().numpy(), orr)


def test_fp16_range():
    """fp16 rows near the top of its range (squares overflow fp16, not fp32) and
    rows of subnormals: the sums are fp32, the outputs rounded once."""
    M, N = 4, 2048
    _, _, x, w, dy = _case(M, N, "f16", seed=9, dy_scale=1.0)
    xs = x.astype(np.float32)
    xs[0] *= 8000.0     # |x| up to ~4e4, x^2 ~ 1e9
    xs[1] *= 1e-6       # mostly subnormal fp16
    xs[2] = 0.0
    x = si.to_storage(xs, "f16")
    assert np.all(np.isfinite(x))
    plain_check(x, w, dy, si.eps_f32(1e-6), "f16", "f16")


@pytest.mark.parametrize("fmt", ALL_FORMATS)
@pytest.mark.parametrize("M,N", [(1, 1), (3, 13), (33, 257), (64, 1024), (31, 4096), (9, 7168), (2, 32768),
                                 (1000, 16)], ids=lambda v: str(v))
def test_residual_small(M, N, fmt):
    _say(f"residual_small M={M} N={N} {fmt}")
    act, wst, x, w, dy = _case(M, N, fmt, seed=3000 + M * 7 + N, dy_scale=1.0 if fmt == "f32" else 1e-2)
    res = si.random_tensor((M, N), act, seed=4000 + M + N)
    dh = si.random_tensor((M, N), act, seed=5000 + M + N, scale=1e-2)
    residual_check(x, res, w, dy, dh, si.eps_f32(1e-5), act, wst)


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_residual_every_ladder_kernel(fmt):
    """Each residual-fused kernel, forced, on ragged shapes with a grid of 2."""
    act = FORMATS[fmt][0]
    epv = 4 if act == "f32" else 8
    for lpr, vpt, wg, pf in _ladder_shapes():
        M, N = _ragged(lpr, vpt, wg, epv)
        cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=lpr, vecs_per_lane=vpt, wg_threads=wg,
                                prefetch=pf, grid=2)
        _say(f"residual kernel lpr={lpr} vpt={vpt} wg={wg} pf={pf} N={N} M={M} {fmt}")
        act, wst, x, w, dy = _case(M, N, fmt, seed=lpr * 10 + vpt + wg + pf)
        res = si.random_tensor((M, N), act, seed=lpr + vpt + 17 * pf)
        dh = si.random_tensor((M, N), act, seed=lpr + vpt + 31 * pf, scale=1e-2)
        residual_check(x, res, w, dy, dh, si.eps_f32(1e-6), act, wst, cfg=cfg)


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_residual_scalar_path(fmt):
    M, N = 37, 1000
    act, wst, x, w, dy = _case(M, N, fmt, seed=79)
    res = si.random_tensor((M, N), act, seed=80)
    dh = si.random_tensor((M, N), act, seed=81, scale=1e-2)
    residual_check(x, res, w, dy, dh, si.eps_f32(1e-5), act, wst, cfg=rn.rmsnorm_config(vector_path=0, grid=5))


def test_residual_equals_unfused():
    """The fused pair equals the unfused composition run on the GPU: y and rstd
    of rmsnorm_fwd(h) bit for bit, and the fused dx equals dh plus the plain
    backward's dx up to that one extra rounding."""
    M, N, act = 256, 4096, "bf16"
    _, _, x, w, dy = _case(M, N, "bf16", seed=82)
    res = si.random_tensor((M, N), act, seed=83)
    dh = si.random_tensor((M, N), act, seed=84, scale=1e-2)
    eps = si.eps_f32(1e-6)
    # one explicit configuration for both paths: the row-sum order and the
    # dW partial-row count are then the same
    cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=256, vecs_per_lane=2, wg_threads=256, prefetch=1,
                            grid=64)
    h, y, rstd = gpu_fwd_residual(x, res, w, eps, act, cfg=cfg)
    y2, rstd2 = gpu_fwd(h, w, eps, act, cfg=cfg)
    assert np.array_equal(y, y2) and np.array_equal(rstd.view(np.uint32), rstd2.view(np.uint32))
    dx, dw = gpu_bwd(h, w, dy, rstd, act, cfg=cfg, dh=dh)
    dx2, dw2 = gpu_bwd(h, w, dy, rstd, act, cfg=cfg)
    assert np.array_equal(dw.view(np.uint32), dw2.view(np.uint32)), "dh must not change dW"
    # fused: round(dh + g); unfused: round(dh + round(g)); they differ by at
    # most one bf16 rounding of the result
    a, b = widen(dx, act), widen(dh, act) + widen(dx2, act)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 2.0 ** -7 * np.abs(widen(dx2, act)) + 1e-30)


def test_residual_null_rstd_and_empty():
    M, N, act = 5, 512, "bf16"
    _, _, x, w, _ = _case(M, N, "bf16", seed=85)
    res = si.random_tensor((M, N), act, seed=86)
    h = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(h)
    rn.rmsnorm_fwd_residual(to_device(x), to_device(res), to_device(w), 1e-5, M, N, rn.BF16, h, y, None)
    torch.cuda.synchronize()
    oh, oy, _ = oracle.fwd_residual(x, res, w, si.eps_f32(1e-5), act)
    assert np.array_equal(widen(to_host(h, act), act), oh)
    check_rows(to_host(y, act), oy, act, "y (no rstd)")
    e = torch.empty((0, N), dtype=torch.bfloat16, device="cuda")
    wd = to_device(w)
    rn.rmsnorm_fwd_residual(e, e, wd, 1e-5, 0, N, rn.BF16, e, e, None)
    dw = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    rn.rmsnorm_bwd_residual(e, wd, e, e, None, 0, N, rn.BF16, e, dw, None, 0)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)


def test_residual_dw_bit_identical_across_reruns():
    M, N, act = 2048, 4096, "bf16"
    _, _, x, w, dy = _case(M, N, "bf16", seed=87)
    res = si.random_tensor((M, N), act, seed=88)
    dh = si.random_tensor((M, N), act, seed=89, scale=1e-2)
    h, _, rstd = gpu_fwd_residual(x, res, w, si.eps_f32(1e-6), act)
    ref_dx, ref = gpu_bwd(h, w, dy, rstd, act, dh=dh)
    for i in range(5):
        _pad = torch.empty(1 + i * 4096, device="cuda")
        dx, dw = gpu_bwd(h, w, dy, rstd, act, dh=dh)
        assert np.array_equal(dw.view(np.uint32), ref.view(np.uint32)), f"dW bits differ on rerun {i}"
        assert np.array_equal(dx, ref_dx), f"dx bits differ on rerun {i}"
        del _pad


def _sample_rows(M, k=32, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(k, M), replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("fmt,M,N", [("bf16", 16384, 4096), ("f16", 16384, 4096), ("bf16w32", 4096, 8192),
                                     ("f16w32", 8192, 5120), ("bf16", 1048576, 128)],
                         ids=lambda v: str(v))
def test_residual_full_size(fmt, M, N):
    """Full-size residual runs in the default launch configuration: sampled rows
    of h, y, dx; sampled rstd; every dW column."""
    _say(f"residual full size {fmt} {M}x{N}: inputs")
    act, wst, x, w, dy = _case(M, N, fmt, seed=6000 + N)
    res = si.random_tensor((M, N), act, seed=6001 + N)
    dh = si.random_tensor((M, N), act, seed=6002 + N, scale=1e-2)
    _say(f"residual full size {fmt} {M}x{N}: gpu + oracle")
    residual_check(x, res, w, dy, dh, si.eps_f32(1e-6), act, wst, rows=_sample_rows(M, seed=N))


@pytest.mark.parametrize("fmt,M,N", [("f16", 16384, 4096), ("bf16w32", 16384, 4096), ("f16w32", 4096, 32768)],
                         ids=lambda v: str(v))
def test_formats_full_size(fmt, M, N):
    _say(f"format full size {fmt} {M}x{N}")
    act, wst, x, w, dy = _case(M, N, fmt, seed=7000 + N)
    eps = si.eps_f32(1e-6)
    y, rstd = gpu_fwd(x, w, eps, act)
    dx, dw = gpu_bwd(x, w, dy, rstd, act)
    rows = _sample_rows(M, seed=N + 1)
    oy, orr = oracle.fwd(x, w, eps, act, rows=rows, wdtype=wst)
    check_rows(y[rows], oy, act, "y")
    check_rstd(rstd[rows], orr)
    odx, orr = oracle.bwd_dx(x, w, dy, eps, act, rows=rows, wdtype=wst)
    check_rows(dx[rows], odx, act, "dx", floor=term_rms(x, w, dy, orr, act, rows=rows))
    check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act)


def _wide_shapes(fmt):
    """(vectors per lane, prefetch) of the wide-row backward kernels built for a format."""
    vpts = range(2, 9) if fmt == "f32" else range(2, 5)
    return [(v, pf) for v in vpts for pf in (0, 1) if not (fmt == "f32" and v >= 6 and pf)]


@pytest.mark.parametrize("fmt", ALL_FORMATS)
@pytest.mark.parametrize("residual", [False, True])
def test_every_wide_kernel(fmt, residual):
    """Each wide-row backward kernel (1024 lanes per row, dW sums in LDS), forced
    on a ragged row (the last vector slot partly empty), 7 rows and a grid of 3
    so workgroups loop over rows and the last one runs short."""
    act, wst, code = FORMATS[fmt]
    epv = 4 if act == "f32" else 8
    for vpt, pf in _wide_shapes(fmt):
        nvec = 1024 * (vpt - 1) + 517
        M, N = 7, nvec * epv
        cfg = rn.rmsnorm_config(vector_path=2, lanes_per_row=1024, vecs_per_lane=vpt, wg_threads=1024,
                                prefetch=pf, grid=3)
        _say(f"wide kernel vpt={vpt} pf={pf} N={N} M={M} {fmt} residual={residual}")
        _, _, x, w, dy = _case(M, N, fmt, seed=9000 + vpt * 10 + pf)
        eps = si.eps_f32(1e-6)
        if residual:
            res = si.random_tensor((M, N), act, seed=9100 + vpt)
            dh = si.random_tensor((M, N), act, seed=9200 + vpt, scale=1e-2)
            h, _, rstd = gpu_fwd_residual(x, res, w, eps, act)
            dx, dw = gpu_bwd(h, w, dy, rstd, act, cfg=cfg, dh=dh)
            odx, orr = oracle.bwd_dx(x, w, dy, eps, act, res=res, dh=dh, wdtype=wst)
            check_rows(dx, odx, act, "dx (wide, residual)", floor=term_rms(h, w, dy, orr, act, dh=dh))
            check_dw(dw, oracle.bwd_dw(x, dy, eps, act, res=res), act, "dW (wide, residual)")
        else:
            _, rstd = gpu_fwd(x, w, eps, act)
            dx, dw = gpu_bwd(x, w, dy, rstd, act, cfg=cfg)
            odx, orr = oracle.bwd_dx(x, w, dy, eps, act, wdtype=wst)
            check_rows(dx, odx, act, "dx (wide)", floor=term_rms(x, w, dy, orr, act))
            check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act, "dW (wide)")
            # same row-sum order and per-lane dW order as the register kernel of
            # the same shape and grid: identical bits
            reg = rn.rmsnorm_config(vector_path=1, lanes_per_row=1024, vecs_per_lane=vpt, wg_threads=1024,
                                    prefetch=0, grid=3)
            dx2, dw2 = gpu_bwd(x, w, dy, rstd, act, cfg=reg)
            assert np.array_equal(dx, dx2) and np.array_equal(dw.view(np.uint32), dw2.view(np.uint32))


@pytest.mark.parametrize("fmt", ALL_FORMATS)
@pytest.mark.parametrize("residual", [False, True])
def test_every_deep_prefetch_kernel_formats(fmt, residual):
    """Depth-2 prefetch backward kernels of every format, plain and residual."""
    act, wst, code = FORMATS[fmt]
    epv = 4 if act == "f32" else 8
    for lpr, wg in ((1, 256), (16, 256), (64, 1024), (256, 1024), (512, 512), (1024, 1024)):
        nvec = max(1, lpr // 2 + 1) if lpr > 1 else 1
        M, N = 5 * (wg // lpr) + 1, nvec * epv
        cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=lpr, vecs_per_lane=1, wg_threads=wg, prefetch=2,
                                grid=2)
        _say(f"deep prefetch lpr={lpr} wg={wg} N={N} M={M} {fmt} residual={residual}")
        _, _, x, w, dy = _case(M, N, fmt, seed=9500 + lpr)
        eps = si.eps_f32(1e-6)
        if residual:
            res = si.random_tensor((M, N), act, seed=9600 + lpr)
            dh = si.random_tensor((M, N), act, seed=9700 + lpr, scale=1e-2)
            h, _, rstd = gpu_fwd_residual(x, res, w, eps, act)
            dx, dw = gpu_bwd(h, w, dy, rstd, act, cfg=cfg, dh=dh)
            odx, orr = oracle.bwd_dx(x, w, dy, eps, act, res=res, dh=dh, wdtype=wst)
            check_rows(dx, odx, act, "dx (deep, residual)", floor=term_rms(h, w, dy, orr, act, dh=dh))
            check_dw(dw, oracle.bwd_dw(x, dy, eps, act, res=res), act, "dW (deep, residual)")
        else:
            _, rstd = gpu_fwd(x, w, eps, act)
            dx, dw = gpu_bwd(x, w, dy, rstd, act, cfg=cfg)
            odx, orr = oracle.bwd_dx(x, w, dy, eps, act, wdtype=wst)
            check_rows(dx, odx, act, "dx (deep)", floor=term_rms(x, w, dy, orr, act))
            check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act, "dW (deep)")


@pytest.mark.parametrize("fmt", ALL_FORMATS)
@pytest.mark.parametrize("residual", [False, True])
def test_every_workgroup_row_kernel_formats(fmt, residual):
    """Backward kernels whose row is the whole workgroup (sized at launch to
    the row's whole wavefronts), every format, plain and residual, both
    prefetch depths; a ragged last wavefront and 7 rows over a grid of 3."""
    act, wst, code = FORMATS[fmt]
    epv = 4 if act == "f32" else 8
    for lanes in (384, 640, 896):
        nvec = lanes - 21
        M, N = 7, nvec * epv
        _, _, x, w, dy = _case(M, N, fmt, seed=9800 + lanes)
        eps = si.eps_f32(1e-6)
        res = si.random_tensor((M, N), act, seed=9900 + lanes)
        dh = si.random_tensor((M, N), act, seed=9950 + lanes, scale=1e-2)
        for pf in (1, 2):
            cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=lanes, vecs_per_lane=1, wg_threads=lanes,
                                    prefetch=pf, grid=3)
            _say(f"workgroup row lanes={lanes} pf={pf} N={N} M={M} {fmt} residual={residual}")
            if residual:
                h, _, rstd = gpu_fwd_residual(x, res, w, eps, act)
                dx, dw = gpu_bwd(h, w, dy, rstd, act, cfg=cfg, dh=dh)
                odx, orr = oracle.bwd_dx(x, w, dy, eps, act, res=res, dh=dh, wdtype=wst)
                check_rows(dx, odx, act, "dx (workgroup row, residual)", floor=term_rms(h, w, dy, orr, act, dh=dh))
                check_dw(dw, oracle.bwd_dw(x, dy, eps, act, res=res), act, "dW (workgroup row, residual)")
            else:
                _, rstd = gpu_fwd(x, w, eps, act)
                dx, dw = gpu_bwd(x, w, dy, rstd, act, cfg=cfg)
                odx, orr = oracle.bwd_dx(x, w, dy, eps, act, wdtype=wst)
                check_rows(dx, odx, act, "dx (workgroup row)", floor=term_rms(x, w, dy, orr, act))
                check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act, "dW (workgroup row)")


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_forward_mid_size_grid(fmt):
    """Mid-size inputs (4 to 8 row blocks of 256 lanes per compute unit): the
    ladder's forward runs a prefetching grid of three 256-lane workgroups per
    CU, or one 1024-lane workgroup per CU walking two blocks, so workgroups
    loop over several row blocks; every row of y and every rstd against the
    oracle. The residual-fused call at the same sizes keeps one block per
    workgroup. Rows of 64 to 256 lanes: 8192 x 512 (16-bit) and 8192 x 256
    (fp32) take the 1024-lane grid in every format."""
    act, wst, code = FORMATS[fmt]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wide_n = 256 if act == "f32" else 512
    for M, N in ((2048, 4096), (4096, 2048), (32 * cus, wide_n)):
        c = rn.rmsnorm_query_config(M, N, code, 0)
        if c.wg_threads == 1024:
            assert (c.grid, c.prefetch, c.rows_per_wg) == (cus, 1, 1024 // c.lanes_per_row), c.as_dict()
        else:
            assert (c.grid, c.prefetch) == (3 * cus, 1), c.as_dict()
        if N == wide_n:
            assert c.wg_threads == 1024, c.as_dict()
        _say(f"mid-size forward {fmt} {M}x{N} wg={c.wg_threads} grid={c.grid}")
        _, _, x, w, dy = _case(M, N, fmt, seed=9990 + M)
        eps = si.eps_f32(1e-6)
        y, rstd = gpu_fwd(x, w, eps, act)
        oy, orr = oracle.fwd(x, w, eps, act, wdtype=wst)
        check_rows(y, oy, act, "y (mid-size grid)")
        check_rstd(rstd, orr)
        res = si.random_tensor((M, N), act, seed=9991 + M)
        h, y2, rstd2 = gpu_fwd_residual(x, res, w, eps, act)
        oh, oy2, orr2 = oracle.fwd_residual(x, res, w, eps, act, wdtype=wst)
        assert np.array_equal(widen(h, act), oh)
        check_rows(y2, oy2, act, "y (residual, mid-size)")
        check_rstd(rstd2, orr2)


@pytest.mark.parametrize("fmt", ["bf16", "f32", "f16"])
def test_forward_narrow_rows_grid(fmt):
    """Rows narrower than a wavefront at 16 row blocks per CU: the ladder's
    prefetching grid of four workgroups per CU, each walking four blocks;
    every row of y and every rstd against the oracle."""
    act, wst, code = FORMATS[fmt]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 64 if act == "f32" else 128  # 16 vectors: 16 lanes, 16 rows per workgroup
    M = 16 * 16 * cus
    c = rn.rmsnorm_query_config(M, N, code, 0)
    assert (c.lanes_per_row, c.grid, c.prefetch) == (16, 4 * cus, 1), c.as_dict()
    _say(f"narrow forward {fmt} {M}x{N} grid={c.grid}")
    _, _, x, w, _ = _case(M, N, fmt, seed=9960)
    eps = si.eps_f32(1e-6)
    y, rstd = gpu_fwd(x, w, eps, act)
    oy, orr = oracle.fwd(x, w, eps, act, wdtype=wst)
    check_rows(y, oy, act, "y (narrow grid)")
    check_rstd(rstd, orr)


@pytest.mark.parametrize("fmt", ["bf16", "f32", "f16"])
def test_forward_explicit_config_keeps_workgroup(fmt):
    """An explicit forward configuration runs on the workgroup it names, also
    where the ladder's grid rules would reshape the ladder's own choice (rows
    of exactly 64 vectors on 512-lane workgroups at 16 row blocks of 256 lanes
    per CU and on 1024-lane ones beyond 20, and mid-size inputs that take one
    1024-lane workgroup per CU): the same rows
    on 256- and on 1024-lane workgroups, each against the oracle, and the
    ladder's own configuration passed back explicitly."""
    act, wst, code = FORMATS[fmt]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 256 if act == "f32" else 512  # 64 vectors: 64 lanes of one vector
    for M in (32 * cus, 64 * cus, 128 * cus):
        _, _, x, w, _ = _case(M, N, fmt, seed=9970 + M)
        eps = si.eps_f32(1e-6)
        oy, orr = oracle.fwd(x, w, eps, act, wdtype=wst)
        lad = rn.rmsnorm_query_config(M, N, code, 0)
        variants = [("ladder", lad)]
        for wg in (256, 1024):
            c = rn.rmsnorm_config(vector_path=1, lanes_per_row=64, vecs_per_lane=1, wg_threads=wg,
                                  prefetch=0, stream_loads=1, grid=-(-M // (wg // 64)))
            variants.append((f"wg{wg}", c))
        for name, c in variants:
            _say(f"explicit forward {fmt} {M}x{N} {name} wg={c.wg_threads} grid={c.grid}")
            y, rstd = gpu_fwd(x, w, eps, act, cfg=c)
            check_rows(y, oy, act, f"y ({name})")
            check_rstd(rstd, orr)


@pytest.mark.parametrize("fmt", ALL_FORMATS)
@pytest.mark.parametrize("residual", [False, True])
def test_every_element_kernel(fmt, residual):
    """The element kernels (rows that are not a multiple of 16 bytes), every
    format, plain and residual, every elements-per-lane count (K = 1..16) on
    1024-lane rows: the ladder's own configuration (its row size is the
    ladder's; it must cover the row), and the 1024-lane kernel forced to a
    grid of 3 so that workgroups walk several rows; 7 rows, of 5 elements
    short of 1024 * K and of one element past 1024 * (K - 1) (only lane 0
    holds an element at k = K - 1)."""
    act, wst, code = FORMATS[fmt]
    eps = si.eps_f32(1e-6)
    for k, N in [(k, n) for k in range(1, 17) for n in (1024 * k - 5, 1024 * (k - 1) + 1) if n >= 257]:
        M = 7
        _, _, x, w, dy = _case(M, N, fmt, seed=7000 + N)
        for d in (0, 1):
            c = rn.rmsnorm_query_config(M, N, code, d)
            assert (c.vector_path, c.elems_per_access, c.prefetch) == (3, 1, 0), c.as_dict()
            assert c.lanes_per_row * c.vecs_per_lane >= N and c.vecs_per_lane <= 16, c.as_dict()
        forced = rn.rmsnorm_config(vector_path=3, lanes_per_row=1024, vecs_per_lane=k, elems_per_access=1,
                                   wg_threads=1024, grid=3)
        for cfg in (None, forced):
            _say(f"element kernel k={k} N={N} {fmt} residual={residual} cfg={None if cfg is None else cfg.as_dict()}")
            if residual:
                res = si.random_tensor((M, N), act, seed=7100 + k)
                dh = si.random_tensor((M, N), act, seed=7200 + k, scale=1e-2)
                residual_check(x, res, w, dy, dh, eps, act, wst, cfg=cfg)
            else:
                plain_check(x, w, dy, eps, act, wst, cfg=cfg)


@pytest.mark.parametrize("fmt", ALL_FORMATS)
@pytest.mark.parametrize("residual", [False, True])
def test_element_kernels_grouped(fmt, residual):
    """Element kernels moving G > 1 consecutive elements per access: rows of
    N = G * (1024 K - 1) columns (G the largest power of two dividing N, so
    the ladder picks G) for the smallest, a middle and the largest K that G
    allows; where G accesses are 16 bytes wide the row is vectorisable and the
    element kernel is forced (elems_per_access = G). The ladder's
    configuration, and the same kernel on a grid of 3 so that workgroups walk
    several rows; 7 rows."""
    act, wst, code = FORMATS[fmt]
    s = 4 if act == "f32" else 2
    big = max(s, 4 if wst == "f32" else 2)
    eps = si.eps_f32(1e-6)
    for g in (2, 4, 8):
        if g * big > 16:
            continue
        kmax = 16 // g
        for k in sorted({1, max(1, kmax // 2), kmax}):
            M, N = 7, g * (1024 * k - 1)
            if N < 257:
                continue
            _, _, x, w, dy = _case(M, N, fmt, seed=7400 + N)
            forced = rn.rmsnorm_config(vector_path=3, lanes_per_row=1024, vecs_per_lane=k, elems_per_access=g,
                                       wg_threads=1024, grid=3)
            if g * s < 16:
                for d in (0, 1):
                    c = rn.rmsnorm_query_config(M, N, code, d)
                    assert (c.vector_path, c.elems_per_access) == (3, g), c.as_dict()
                    assert c.lanes_per_row * c.vecs_per_lane * g >= N, c.as_dict()
                cfgs = (None, forced)
            else:
                ladder = rn.rmsnorm_config(vector_path=3, lanes_per_row=1024, vecs_per_lane=k, elems_per_access=g,
                                           wg_threads=1024, grid=M)
                cfgs = (ladder, forced)
            for cfg in cfgs:
                _say(f"grouped element kernel g={g} k={k} N={N} {fmt} residual={residual} "
                     f"cfg={None if cfg is None else cfg.as_dict()}")
                if residual:
                    res = si.random_tensor((M, N), act, seed=7500 + N)
                    dh = si.random_tensor((M, N), act, seed=7600 + N, scale=1e-2)
                    residual_check(x, res, w, dy, dh, eps, act, wst, cfg=cfg)
                else:
                    plain_check(x, w, dy, eps, act, wst, cfg=cfg)


@pytest.mark.parametrize("fmt", ALL_FORMATS)
@pytest.mark.parametrize("residual", [False, True])
def test_element_kernels_every_row_size(fmt, residual):
    """Element rows of 64, 128, 256 and 512 lanes (1024 above), one and G > 1
    elements per access, the fewest and the most accesses per lane: rows of
    N = G * (lanes * K - 1) columns forced onto that kernel with a grid of 3
    (workgroups walk several rows); 7 rows, plain and residual, against the
    oracle."""
    act, wst, code = FORMATS[fmt]
    big = max(4 if act == "f32" else 2, 4 if wst == "f32" else 2)
    eps = si.eps_f32(1e-6)
    for lanes in (64, 128, 256, 512):
        for g in (1, 2, 4):
            if g * big > 16:
                continue
            for k in (1, 16 // g):
                M, N = 7, g * (lanes * k - 1)
                _, _, x, w, dy = _case(M, N, fmt, seed=7700 + N + lanes)
                cfg = rn.rmsnorm_config(vector_path=3, lanes_per_row=lanes, vecs_per_lane=k, elems_per_access=g,
                                        wg_threads=lanes, grid=3)
                _say(f"element rows lanes={lanes} g={g} k={k} N={N} {fmt} residual={residual}")
                if residual:
                    res = si.random_tensor((M, N), act, seed=7800 + N)
                    dh = si.random_tensor((M, N), act, seed=7900 + N, scale=1e-2)
                    residual_check(x, res, w, dy, dh, eps, act, wst, cfg=cfg)
                else:
                    plain_check(x, w, dy, eps, act, wst, cfg=cfg)


@pytest.mark.parametrize("fmt,off", [("bf16", 1), ("bf16", 2), ("bf16", 4), ("f32", 1), ("f32", 2),
                                     ("f16w32", 1), ("f16w32", 2)])
def test_element_kernels_on_unaligned_pointers(fmt, off):
    """16-byte-multiple rows whose pointers are not 16-byte aligned (views
    `off` elements into larger buffers: 2- to 8-byte alignment, so one to four
    elements per access) take the element kernels; outputs against the
    oracle, and nothing written outside the views."""
    act, wst, code = FORMATS[fmt]
    M, N = 37, 4096
    _, _, x, w, dy = _case(M, N, fmt, seed=7300 + off)
    eps = si.eps_f32(1e-6)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[act]

    def view_of(a, dtype):
        d = to_device(np.concatenate([a.reshape(-1)[:off], a.reshape(-1)]), dtype)
        return d[off:]

    xd, dyd = view_of(x, act), view_of(dy, act)
    wd = view_of(w, wst)
    ybuf = torch.full((M * N + 2 * off,), float("nan"), dtype=tdt, device="cuda")
    dxbuf = torch.full((M * N + 2 * off,), float("nan"), dtype=tdt, device="cuda")
    y, dx = ybuf[off:M * N + off], dxbuf[off:M * N + off]
    assert y.data_ptr() % 16 != 0 and xd.data_ptr() % 16 != 0
    rstd = torch.full((M,), float("nan"), device="cuda")
    dw = torch.full((N,), float("nan"), device="cuda")
    _say(f"unaligned element kernels {fmt} off={off}")
    rn.rmsnorm_fwd(xd, wd, eps, M, N, code, y, rstd)
    nb = rn.rmsnorm_bwd_workspace_bytes(M, N, code)
    ws = torch.empty(nb // 4 + 64, device="cuda")
    rn.rmsnorm_bwd(xd, wd, dyd, rstd, M, N, code, dx, dw, ws, nb)
    torch.cuda.synchronize()
    assert torch.isnan(ybuf[:off]).all() and torch.isnan(ybuf[M * N + off:]).all()
    assert torch.isnan(dxbuf[:off]).all() and torch.isnan(dxbuf[M * N + off:]).all()
    oy, orr = oracle.fwd(x, w, eps, act, wdtype=wst)
    check_rows(to_host(y, act).reshape(M, N), oy, act, "y (unaligned)")
    check_rstd(rstd.cpu().numpy(), orr)
    odx, orr = oracle.bwd_dx(x, w, dy, eps, act, wdtype=wst)
    check_rows(to_host(dx, act).reshape(M, N), odx, act, "dx (unaligned)", floor=term_rms(x, w, dy, orr, act))
    check_dw(dw.cpu().numpy(), oracle.bwd_dw(x, dy, eps, act), act)
