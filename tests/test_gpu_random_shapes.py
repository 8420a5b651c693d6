"""Seeded random shapes through the ladder: every kernel family the ladder can
pick (narrow rows several to a wavefront, power-of-two and whole-wavefront
rows, wide rows with LDS sums, the mid-size forward grid, the single-workgroup
backward, the element kernels for rows of 257 to 16384 columns that are not a
multiple of 16 bytes, and the scalar path for the other such rows) in
every storage format, plain and with the fused residual add, against the fp64
oracle. The cases are drawn once from a fixed seed, so a failure names a case
that reproduces."""

from __future__ import annotations

import sys
import zlib

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
                         gpu_fwd_residual, term_rms, widen)


def _cases(n=48, seed=20261202, max_elems=3 << 20):
    rng = np.random.default_rng(seed)
    widths = [8, 64, 96, 128, 1000, 1024, 2560, 3072, 4096, 4104, 5120, 6144, 7168, 8192, 12288, 16384, 20480,
              24576, 32768, 13, 257, 4095, 5001]
    out = []
    while len(out) < n:
        N = int(rng.choice(widths)) if rng.random() < 0.8 else int(rng.integers(1, 40000))
        M = int(rng.choice([1, 2, 7, 16, 33, 256, 1000, 2048, 4096])) if rng.random() < 0.7 else int(rng.integers(1, 5000))
        if M * N > max_elems:
            M = max(1, max_elems // N)
        fmt = str(rng.choice(list(FORMATS)))
        residual = bool(rng.random() < 0.3)
        out.append((M, N, fmt, residual))
    return out


# Fixed cases for the families a random draw rarely reaches: whole-wavefront
# backward rows (320, 384, 640 and 768 lanes), the mid-size forward grid, the
# element kernels at 2 and 4 elements per access (4100 and 4098 columns; the
# 16-bit forward on a resident grid), the resident forward grid of fp32
# weights (more than 8 row blocks per compute unit), and rows wider than a
# workgroup: split-row backwards of 3 to 13 members (two per CU for 16-bit
# rows, one per CU for fp32), the two-pass forward (plain and residual), and
# an unvectorisable row beyond the element kernels (the scalar kernels).
CASES = _cases() + [(2048, 2560, "bf16", False), (1000, 3072, "f16", True), (600, 5120, "bf16", False),
                    (500, 6144, "f16", True), (2048, 4096, "f16", False), (4096, 2048, "bf16w32", False),
                    (3000, 4100, "bf16", False), (777, 4098, "f32", True), (1500, 2050, "bf16w32", False),
                    (4500, 4096, "f16w32", False),
                    (40, 36864, "f32", False), (20, 49160, "bf16", False), (12, 131080, "f16", True),
                    (6, 200000, "bf16w32", False), (5, 70000, "f32", True), (3, 300001, "f32", False)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("M,N,fmt,residual", CASES, ids=[f"{m}x{n}-{f}{'-res' if r else ''}" for m, n, f, r in CASES])
def test_random_shape(M, N, fmt, residual):
    act, wst, code = FORMATS[fmt]
    seed = (M * 1_000_003 + N * 7 + zlib.crc32(fmt.encode()) % 97) % (1 << 31)  # str hash() varies per process
    x, w, dy = si.random_case(M, N, act, seed=seed, dy_scale=1.0 if act == "f32" else 1e-2, wdtype=wst)
    eps = si.eps_f32(1e-6)
    fc, bc = rn.rmsnorm_query_config(M, N, code, 0), rn.rmsnorm_query_config(M, N, code, 1)
    _say(f"random {M}x{N} {fmt} residual={residual} fwd={fc.as_dict()} bwd={bc.as_dict()}")
    if residual:
        res = si.random_tensor((M, N), act, seed=seed + 1)
        dh = si.random_tensor((M, N), act, seed=seed + 2, scale=1e-2)
        h, y, rstd = gpu_fwd_residual(x, res, w, eps, act)
        oh, oy, orr = oracle.fwd_residual(x, res, w, eps, act, wdtype=wst)
        assert np.array_equal(widen(h, act), oh), "h differs from round(x + res)"
        check_rows(y, oy, act, "y (residual)")
        check_rstd(rstd, orr)
        dx, dw = gpu_bwd(h, w, dy, rstd, act, dh=dh)
        odx, orr = oracle.bwd_dx(x, w, dy, eps, act, res=res, dh=dh, wdtype=wst)
        check_rows(dx, odx, act, "dx (residual)", floor=term_rms(h, w, dy, orr, act, dh=dh))
        check_dw(dw, oracle.bwd_dw(x, dy, eps, act, res=res), act, "dW (residual)")
    else:
        y, rstd = gpu_fwd(x, w, eps, act)
        oy, orr = oracle.fwd(x, w, eps, act, wdtype=wst)
        check_rows(y, oy, act, "y")
        check_rstd(rstd, orr)
        dx, dw = gpu_bwd(x, w, dy, rstd, act)
        odx, orr = oracle.bwd_dx(x, w, dy, eps, act, wdtype=wst)
        check_rows(dx, odx, act, "dx", floor=term_rms(x, w, dy, orr, act))
        check_dw(dw, oracle.bwd_dw(x, dy, eps, act), act)
    assert np.all(np.isfinite(widen(y, act))) and np.all(np.isfinite(widen(dx, act)))
