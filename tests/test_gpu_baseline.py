"""GPU parity of the unfused reference kernels (include/rmsnorm_baseline.h).

They are measured beside the fused path, so they must compute the same values:
the same oracle gates as the fused kernels, the separate add bit for bit
against the oracle's rounded sum, and the unfused residual composition against
the fused residual calls.
"""

from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import memory_bound_normalization_rmsnorm_amd as rn  # noqa: E402
import oracle  # noqa: E402
import synthetic_inputs as si  # noqa: E402
from parity_util import (FORMATS, check_dw, check_rows, check_rstd, empty_like_storage, gpu_bwd,  # noqa: E402
                         gpu_fwd_residual, term_rms, to_device, to_host, widen)


def unfused_fwd(x, w, eps, act, code):
    M, N = x.shape
    y = empty_like_storage((M, N), act)
    rstd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    rn.rmsn_unfused_fwd(to_device(x), to_device(w), eps, M, N, code, y, rstd)
    torch.cuda.synchronize()
    return to_host(y, act), rstd.cpu().numpy()


def unfused_bwd(x, w, dy, rstd, act, code):
    M, N = x.shape
    dx = empty_like_storage((M, N), act)
    dw = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = rn.rmsn_unfused_bwd_workspace_bytes(M, N, code)
    ws = torch.empty(max(nbytes, 256) // 4, dtype=torch.float32, device="cuda")
    rn.rmsn_unfused_bwd(to_device(x), to_device(w), to_device(dy),
                        torch.from_numpy(np.ascontiguousarray(rstd, np.float32)).cuda(), M, N, code, dx, dw, ws,
                        nbytes)
    torch.cuda.synchronize()
    return to_host(dx, act), dw.cpu().numpy()


SHAPES = [(1, 8), (7, 64), (33, 264), (129, 1000), (64, 4096), (3, 32768), (1000, 16), (300, 128), (517, 5120)]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("M,N", SHAPES, ids=lambda v: str(v))
def test_unfused_matches_oracle(M, N, fmt):
    act, wst, code = FORMATS[fmt]
    print(f"unfused M={M} N={N} {fmt}", flush=True)
    x, w, dy = si.random_case(M, N, act, seed=8000 + M + N, dy_scale=1.0 if act == "f32" else 1e-2, wdtype=wst)
    eps = si.eps_f32(1e-5)
    y, rstd = unfused_fwd(x, w, eps, act, code)
    oy, orr = oracle.fwd(x, w, eps, act, wdtype=wst)
    check_rows(y, oy, act, "y (unfused)")
    check_rstd(rstd, orr)
    dx, dw = unfused_bwd(x, w, dy, rstd, act, code)
    odx, orr = oracle.bwd_dx(x, w, dy, eps, act, wdtype=wst)
    check_rows(dx, odx, act, "dx (unfused)", floor=term_rms(x, w, dy, orr, act))
    check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act, "dW (unfused)")
    dx2, dw2 = unfused_bwd(x, w, dy, rstd, act, code)
    assert np.array_equal(dw.view(np.uint32), dw2.view(np.uint32)) and np.array_equal(dx, dx2)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "f16"])
def test_add_bit_exact(fmt):
    """c = round(a + b): bit for bit the oracle's stored residual sum."""
    act = FORMATS[fmt][0]
    M, N = 37, 1024
    a = si.random_tensor((M, N), act, seed=11)
    b = si.random_tensor((M, N), act, seed=12, scale=3.0)
    c = empty_like_storage((M, N), act)
    rn.rmsn_add(to_device(a), to_device(b), c, M * N, FORMATS[fmt][2])
    torch.cuda.synchronize()
    w = si.to_storage(np.ones(N, np.float32), act)
    oh, _, _ = oracle.fwd_residual(a, b, w, 1e-5, act, want_y=False)
    assert np.array_equal(widen(to_host(c, act), act), oh)
    # in place: c aliases a
    ad = to_device(a)
    rn.rmsn_add(ad, to_device(b), ad, M * N, FORMATS[fmt][2])
    torch.cuda.synchronize()
    assert np.array_equal(widen(to_host(ad, act), act), oh)


@pytest.mark.parametrize("fmt", ["bf16", "f16w32"])
def test_unfused_residual_composition(fmt):
    """add then rmsnorm_fwd gives the fused forward's h, y, rstd bit for bit (same
    launch configuration); rmsnorm_bwd then add gives the fused dx up to the
    one extra rounding of the unfused sum."""
    act, wst, code = FORMATS[fmt]
    M, N = 256, 4096
    x, w, dy = si.random_case(M, N, act, seed=90, dy_scale=1e-2, wdtype=wst)
    res = si.random_tensor((M, N), act, seed=91)
    dh = si.random_tensor((M, N), act, seed=92, scale=1e-2)
    eps = si.eps_f32(1e-6)
    cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=256, vecs_per_lane=2, wg_threads=256, prefetch=1, grid=64)
    h, y, rstd = gpu_fwd_residual(x, res, w, eps, act, cfg=cfg)

    hd = empty_like_storage((M, N), act)
    rn.rmsn_add(to_device(x), to_device(res), hd, M * N, code)
    y2 = empty_like_storage((M, N), act)
    r2 = torch.empty(M, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd_with_config(hd, to_device(w), eps, M, N, code, y2, r2, cfg)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(hd, act), h)
    assert np.array_equal(to_host(y2, act), y)
    assert np.array_equal(r2.cpu().numpy().view(np.uint32), rstd.view(np.uint32))

    dx_f, dw_f = gpu_bwd(h, w, dy, rstd, act, cfg=cfg, dh=dh)
    dx_p, dw_p = gpu_bwd(h, w, dy, rstd, act, cfg=cfg)
    assert np.array_equal(dw_f.view(np.uint32), dw_p.view(np.uint32))
    dxd = to_device(dx_p)
    rn.rmsn_add(dxd, to_device(dh), dxd, M * N, code)
    torch.cuda.synchronize()
    a, b = widen(dx_f, act), widen(to_host(dxd, act), act)
    ulp = 2.0 ** -7 if act == "bf16" else 2.0 ** -10
    assert np.all(np.abs(a - b) <= ulp * (np.abs(b) + np.abs(widen(dx_p, act))) + 1e-30)


def test_unfused_bwd_empty_sets_zero():
    N = 64
    dw = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    rn.rmsn_unfused_bwd(None, None, None, None, 0, N, rn.BF16, None, dw, None, 0)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)
