"""rmsnorm_bwd_noalloc (the backward whose dW partial rows live in the
library's static device array) against rmsnorm_bwd (the same kernels with a
caller's workspace), through the C ABI.

Both run the same row kernel on the same grid and the same combine, so dx and
dW must agree bit for bit. Each case makes two calls in a row, the second on
a smaller input, so the second call finds the array holding the first call's
partial rows; every output is poisoned with NaN before each call. The first
outputs are also checked against the fp64 oracle. Shapes cover the vector
kernels with a combine, the single-workgroup call that writes dW itself, the
wide-row kernel at the array's exact limit, the element kernels, M = 0, and
split rows (exchange slots after the partial rows, zeroed by each call). A
shape whose workspace exceeds the array is refused before any launch.
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
from parity_util import (DT, check_dw, check_rows, empty_like_storage, term_rms, to_device,  # noqa: E402
                         to_host, widen)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(M, N, dtype, seed):
    x, w, dy = si.random_case(M, N, dtype, seed=seed, dy_scale=1e-2 if dtype != "f32" else 1.0)
    eps = si.eps_f32(1e-6)
    code = DT[dtype]
    xd, wd, dyd = to_device(x), to_device(w), to_device(dy)
    rstd = torch.empty(max(M, 1), dtype=torch.float32, device="cuda")
    if M > 0:
        y = empty_like_storage((M, N), dtype)
        rn.rmsnorm_fwd(xd, wd, eps, M, N, code, y, rstd)
    return (x, w, dy, eps), (xd, wd, dyd, rstd)


def _run_both(M, N, dtype, dev):
    xd, wd, dyd, rstd = dev
    code = DT[dtype]
    out = {}
    for which in ("noalloc", "workspace"):
        dx = empty_like_storage((max(M, 1), N), dtype)
        dw = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        if which == "noalloc":
            rn.rmsnorm_bwd_noalloc(xd, wd, dyd, rstd, M, N, code, dx, dw)
        else:
            ws_bytes = max(rn.rmsnorm_bwd_workspace_bytes(M, N, code), 256)
            ws = torch.full((ws_bytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
            rn.rmsnorm_bwd(xd, wd, dyd, rstd, M, N, code, dx, dw, ws, ws_bytes)
        torch.cuda.synchronize()
        out[which] = (to_host(dx[:M], dtype), dw.cpu().numpy())
    return out


def _assert_same(out, M, N, dtype):
    (dx_a, dw_a), (dx_b, dw_b) = out["noalloc"], out["workspace"]
    assert np.isfinite(dw_a).all(), "noalloc dW has unwritten (NaN) columns"
    assert np.array_equal(dw_a.view(np.uint32), dw_b.view(np.uint32)), "dW differs from rmsnorm_bwd"
    if M > 0:
        assert np.isfinite(widen(dx_a, dtype)).all(), "noalloc dx has unwritten elements"
        assert np.array_equal(dx_a.view(np.uint8), dx_b.view(np.uint8)), "dx differs from rmsnorm_bwd"


# (first shape, second, smaller shape, format)
PAIRS = [
    ((16384, 4096), (300, 4096), "bf16"),     # depth-2 row kernel + combine, then a smaller grid
    ((4096, 32768), (64, 8192), "bf16"),      # wide-row kernel at exactly 32 MiB of partial rows
    ((1024, 4096), (2, 4096), "f32"),         # combine, then one workgroup writing dW itself
    ((2048, 4100), (33, 257), "bf16"),        # element kernels
    ((777, 2560), (0, 2560), "f16"),          # whole-wavefront rows, then M = 0 (dW = 0)
    ((100, 65536), (2, 49152), "bf16"),       # split rows: exchange slots after the partial rows
]


@pytest.mark.parametrize("first,second,dtype", PAIRS, ids=[f"{a[0]}x{a[1]}-{b[0]}x{b[1]}-{d}" for a, b, d in PAIRS])
def test_noalloc_matches_workspace_call(first, second, dtype):
    for k, (M, N) in enumerate((first, second)):
        _say(f"noalloc {dtype} {M}x{N} (call {k + 1} of 2)")
        host, dev = _case(M, N, dtype, seed=7000 + 31 * k + M % 97)
        out = _run_both(M, N, dtype, dev)
        _assert_same(out, M, N, dtype)
        if k == 0:
            # the first call's outputs against the oracle on a few rows and every dW column
            x, w, dy, eps = host
            rows = np.unique(np.linspace(0, M - 1, 12).astype(np.int64))
            odx, orr = oracle.bwd_dx(x, w, dy, eps, dtype, rows=rows)
            check_rows(out["noalloc"][0][rows], odx, dtype, "dx",
                       floor=term_rms(x, w, dy, orr, dtype, rows=rows))
            check_dw(out["noalloc"][1], oracle.bwd_dw(x, dy, eps, dtype), dtype)
        elif M == 0:
            assert not out["noalloc"][1].any(), "M = 0 must give dW = 0"


def test_noalloc_refuses_shapes_beyond_the_array():
    # bf16 rows of 65536 columns split over two workgroups, one group per two
    # CUs: 128 partial rows of 256 KiB (32 MiB) plus the exchange slots > 32
    # MiB. Refused before any launch.
    M, N = 4096, 65536
    cfg = rn.rmsnorm_query_config(M, N, rn.BF16, 1)
    assert cfg.vector_path == 4
    assert cfg.partial_rows * cfg.partial_stride * 4 + cfg.grid * 16 > rn.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(N, dtype=torch.bfloat16, device="cuda")
    rstd = torch.ones(M, dtype=torch.float32, device="cuda")
    dx = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dw = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(rn.RmsnormError) as e:
        rn.rmsnorm_bwd_noalloc(x, w, x, rstd, M, N, rn.BF16, dx, dw)
    assert e.value.status == rn.ESCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(dx).all() and torch.isnan(dw).all(), "a refused call must launch nothing"
