"""Pins for the fp64 CPU oracle: checks against facts other than the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` handle and raises
``AssertionError`` when the oracle disagrees with

  * the values the hello-gpu chapter 13 page prints for its worked examples
    (section 13.1 and Figure 13.1; fixture ``golden/hello_gpu_ch13_worked_examples.json``),
  * closed forms of the definition (one column, constant rows, zero rows,
    zero weight, the epsilon-dependent scaling ratio),
  * invariants stated on the page (section 13.4: zero input and zero weight
    give zero output; scaling x is exact only without epsilon) or derived
    from the definition (unit mean square of the output, dx orthogonal to x),
  * central finite differences of the forward (pins dx and dW, whose formulas
    are lost on the persistent-backward page),
  * PyTorch's own fp64 ``rms_norm`` and autograd on the CPU, an independent
    implementation of the same definition.

The functions are shared by ``test_oracle.py`` (the real oracle must pass all
of them) and ``test_oracle_mutants.py`` (every planted mistake must fail at
least one of them).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hello_gpu_ch13_worked_examples.json")


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def _f64(v):
    return np.asarray(v, dtype=np.float64)


def _eps32(e):
    return float(np.float32(e))


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e} (bound {bound.max():.3e})"


def pin_worked_examples(orc):
    """hello-gpu ch. 13, section 13.1 and Figure 13.1: printed r and y values."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = _f32([c["x"]])
        w = _f32(c["w"])
        eps = _eps32(c["eps"])
        y, r = orc.fwd(x, w, eps, "f32")
        tol = c["tol"]
        assert abs(r[0] - c["r"]) <= tol, f"r {r[0]} vs printed {c['r']}"
        for j, v in c["y"].items():
            assert abs(y[0, int(j)] - v) <= tol, f"y[{j}] {y[0, int(j)]} vs printed {v}"
        # the printed mean of squares, recovered from r: 1/r^2 - eps
        ms = 1.0 / r[0] ** 2 - eps
        assert abs(ms - c["mean_square"]) <= 1e-9 * c["mean_square"], f"mean square {ms}"


def pin_one_column(orc):
    """N = 1: y = x w / sqrt(x^2 + eps) and dy/dx = dy w eps / (x^2 + eps)^(3/2).

    With x = 1e-3 and eps = 1e-5 the answer depends strongly on where eps
    enters (inside the root: 0.3015...; outside: ~0.99).
    """
    for xv, wv, dyv, eps in [(1e-3, 1.0, 1.0, 1e-5), (-2.5, 0.75, 0.3, 1e-2), (7.0, -1.5, -2.0, 0.5)]:
        x = _f64([[xv]])
        w = _f64([wv])
        dy = _f64([[dyv]])
        y, r = orc.fwd(x, w, eps, "f64")
        expect_y = xv * wv / math.sqrt(xv * xv + eps)
        _close(y[0, 0], expect_y, 1e-14, what="N=1 y")
        dx, _ = orc.bwd_dx(x, w, dy, eps, "f64")
        expect_dx = dyv * wv * eps / (xv * xv + eps) ** 1.5
        _close(dx[0, 0], expect_dx, 1e-12, atol=1e-300, what="N=1 dx")
        dw = orc.bwd_dw(x, dy, eps, "f64")
        _close(dw[0], dyv * xv / math.sqrt(xv * xv + eps), 1e-14, what="N=1 dW")


def pin_constant_rows(orc):
    """Row of N copies of c: r = 1/sqrt(c^2+eps); with constant dy = d and w = 1,
    dx_j = d eps / (c^2+eps)^(3/2). Any denominator other than the true N fails."""
    for N, c, d, eps in [(13, 0.5, 2.0, 1e-2), (257, -3.0, 0.25, 1e-1), (4096, 1.25, -1.0, 1e-5)]:
        x = np.full((1, N), c, dtype=np.float64)
        w = np.linspace(0.5, 1.5, N)
        y, r = orc.fwd(x, w, eps, "f64")
        _close(r[0], 1.0 / math.sqrt(c * c + eps), 1e-14, what="constant row r")
        _close(y[0], c * w / math.sqrt(c * c + eps), 1e-13, what="constant row y")
        dy = np.full((1, N), d, dtype=np.float64)
        dx, _ = orc.bwd_dx(x, np.ones(N), dy, eps, "f64")
        _close(dx[0], np.full(N, d * eps / (c * c + eps) ** 1.5), 1e-9, what="constant row dx")


def pin_zero_cases(orc):
    """hello-gpu ch. 13, section 13.4: zero input -> zero output; zero weight ->
    zero output. Derived: zero weight -> zero dx; zero dy -> zero dx and dW;
    a zero row has r = 1/sqrt(eps)."""
    rng = np.random.default_rng(7)
    M, N, eps = 3, 11, 1e-5
    x = rng.standard_normal((M, N))
    x[1] = 0.0
    w = rng.standard_normal(N)
    dy = rng.standard_normal((M, N))
    y, r = orc.fwd(x, w, eps, "f64")
    assert np.all(y[1] == 0.0), "zero row must give zero output"
    _close(r[1], 1.0 / math.sqrt(eps), 1e-14, what="zero-row r")
    y0, _ = orc.fwd(x, np.zeros(N), eps, "f64")
    assert np.all(y0 == 0.0), "zero weight must give zero output"
    dx0, _ = orc.bwd_dx(x, np.zeros(N), dy, eps, "f64")
    assert np.all(dx0 == 0.0), "zero weight must give zero dx"
    dxz, _ = orc.bwd_dx(x, w, np.zeros((M, N)), eps, "f64")
    assert np.all(dxz == 0.0), "zero dy must give zero dx"
    assert np.all(orc.bwd_dw(x, np.zeros((M, N)), eps, "f64") == 0.0), "zero dy must give zero dW"


def pin_unit_mean_square(orc):
    """With w = 1 and eps = 0 every output row has mean square exactly 1."""
    rng = np.random.default_rng(11)
    for M, N in [(4, 13), (3, 257), (2, 4096)]:
        x = rng.standard_normal((M, N)) * rng.uniform(0.1, 10.0, (M, 1))
        y, _ = orc.fwd(x, np.ones(N), 0.0, "f64")
        _close(np.mean(y * y, axis=1), np.ones(M), 1e-13, what="mean square of y")


def pin_scaling(orc):
    """hello-gpu ch. 13, section 13.4: scaling x is exact only without eps.
    At eps = 0, y(c x) = y(x). With eps > 0 the closed form is
    y(c x) = y(x) * c sqrt(ms + eps) / sqrt(c^2 ms + eps), ms = mean(x^2)."""
    rng = np.random.default_rng(13)
    M, N = 5, 37
    x = rng.standard_normal((M, N))
    w = rng.uniform(0.5, 1.5, N)
    for c in (2.0, 0.01, -3.0):
        y1, _ = orc.fwd(x, w, 0.0, "f64")
        y2, _ = orc.fwd(c * x, w, 0.0, "f64")
        _close(y2, np.sign(c) * y1, 1e-13, atol=1e-15, what="eps=0 scale invariance")
        eps = 1e-2
        y1, _ = orc.fwd(x, w, eps, "f64")
        y2, _ = orc.fwd(c * x, w, eps, "f64")
        ms = np.mean(x * x, axis=1, keepdims=True)
        ratio = c * np.sqrt(ms + eps) / np.sqrt(c * c * ms + eps)
        _close(y2, y1 * ratio, 1e-12, atol=1e-15, what="eps>0 scaling closed form")


def _loss(orc, x, w, dy, eps):
    y, _ = orc.fwd(x, w, eps, "f64")
    return float(np.sum(dy * y))


def pin_finite_differences(orc):
    """Central differences of L = sum(dy * y(x, w)) match dx and dW."""
    rng = np.random.default_rng(17)
    for M, N, eps in [(1, 1, 1e-3), (2, 3, 1e-5), (4, 8, 1e-2), (3, 5, 0.0)]:
        x = rng.standard_normal((M, N))
        w = rng.uniform(0.5, 1.5, N)
        dy = rng.standard_normal((M, N))
        dx, _ = orc.bwd_dx(x, w, dy, eps, "f64")
        dw = orc.bwd_dw(x, dy, eps, "f64")
        fdx = np.empty_like(x)
        for i in range(M):
            for j in range(N):
                h = 1e-6 * max(1.0, abs(x[i, j]))
                xp = x.copy()
                xm = x.copy()
                xp[i, j] += h
                xm[i, j] -= h
                fdx[i, j] = (_loss(orc, xp, w, dy, eps) - _loss(orc, xm, w, dy, eps)) / (2 * h)
        fdw = np.empty(N)
        for j in range(N):
            h = 1e-6 * max(1.0, abs(w[j]))
            wp = w.copy()
            wm = w.copy()
            wp[j] += h
            wm[j] -= h
            fdw[j] = (_loss(orc, x, wp, dy, eps) - _loss(orc, x, wm, dy, eps)) / (2 * h)
        scale_x = max(1.0, np.max(np.abs(fdx)))
        scale_w = max(1.0, np.max(np.abs(fdw)))
        _close(dx, fdx, 0.0, atol=1e-7 * scale_x, what=f"dx vs finite differences {M}x{N}")
        _close(dw, fdw, 0.0, atol=1e-7 * scale_w, what=f"dW vs finite differences {M}x{N}")


def pin_backward_closed_forms(orc):
    """Derived from the definition:
    * eps = 0: sum_j x_ij dx_ij = 0 (dx is orthogonal to x);
    * dW_j = sum_i dy_ij y_ij / w_j;
    * one row: dW = dy * x * r;
    * eps = 0: dx(c x) = dx(x) / c.
    """
    rng = np.random.default_rng(19)
    M, N = 6, 29
    x = rng.standard_normal((M, N))
    w = rng.uniform(0.5, 1.5, N)
    dy = rng.standard_normal((M, N))
    dx, _ = orc.bwd_dx(x, w, dy, 0.0, "f64")
    dots = np.sum(x * dx, axis=1)
    norms = np.linalg.norm(x, axis=1) * np.linalg.norm(dx, axis=1)
    assert np.all(np.abs(dots) <= 1e-13 * norms), f"x.dx not zero: {np.max(np.abs(dots) / norms):.3e}"
    eps = 1e-3
    y, r = orc.fwd(x, w, eps, "f64")
    dw = orc.bwd_dw(x, dy, eps, "f64")
    _close(dw, np.sum(dy * y, axis=0) / w, 1e-12, atol=1e-14, what="dW = sum(dy*y)/w")
    dw1 = orc.bwd_dw(x[2:3], dy[2:3], eps, "f64")
    _close(dw1, dy[2] * x[2] * r[2], 1e-14, what="one-row dW")
    c = 3.5
    dxc, _ = orc.bwd_dx(c * x, w, dy, 0.0, "f64")
    _close(dxc, dx / c, 1e-12, atol=1e-15, what="dx homogeneity")


def pin_torch_reference(orc):
    """PyTorch CPU fp64 rms_norm and autograd (an independent implementation of
    the same definition) agree with the oracle, on the page's boundary shapes
    3x13 and 33x257 (hello-gpu ch. 13, section 13.4)."""
    import torch

    rng = np.random.default_rng(23)
    for M, N, eps in [(3, 13, 1e-5), (33, 257, 1e-6), (5, 64, 0.1)]:
        x = rng.standard_normal((M, N))
        w = rng.uniform(0.5, 1.5, N)
        dy = rng.standard_normal((M, N))
        xt = torch.tensor(x, requires_grad=True)
        wt = torch.tensor(w, requires_grad=True)
        yt = torch.nn.functional.rms_norm(xt, (N,), wt, eps)
        yt.backward(torch.tensor(dy))
        y, _ = orc.fwd(x, w, eps, "f64")
        dx, _ = orc.bwd_dx(x, w, dy, eps, "f64")
        dw = orc.bwd_dw(x, dy, eps, "f64")
        _close(y, yt.detach().numpy(), 1e-13, atol=1e-15, what="y vs torch")
        _close(dx, xt.grad.numpy(), 1e-11, atol=1e-13, what="dx vs torch")
        _close(dw, wt.grad.numpy(), 1e-11, atol=1e-13, what="dW vs torch")


def pin_storage_widening(orc):
    """bf16 and fp32 storage widen exactly: the oracle on bf16 bit patterns or
    fp32 values equals the oracle on the same numbers stored as fp64."""
    rng = np.random.default_rng(29)
    M, N, eps = 4, 24, 1e-5
    x32 = rng.standard_normal((M, N)).astype(np.float32)
    w32 = rng.uniform(0.5, 1.5, N).astype(np.float32)
    dy32 = rng.standard_normal((M, N)).astype(np.float32)
    # bf16 patterns by truncation (exactly representable by construction)
    def trunc(a):
        return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)

    def widen(b):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)

    xb, wb, dyb = trunc(x32), trunc(w32), trunc(dy32)
    for args, dt in [((x32, w32, dy32), "f32"), ((xb, wb, dyb), "bf16")]:
        x, w, dy = args
        if dt == "f32":
            x64, w64, dy64 = x.astype(np.float64), w.astype(np.float64), dy.astype(np.float64)
        else:
            x64, w64, dy64 = widen(x), widen(w), widen(dy)
        y, r = orc.fwd(x, w, eps, dt)
        y64, r64 = orc.fwd(x64, w64, eps, "f64")
        assert np.array_equal(y, y64) and np.array_equal(r, r64), f"{dt} forward widening"
        dx, _ = orc.bwd_dx(x, w, dy, eps, dt)
        dx64, _ = orc.bwd_dx(x64, w64, dy64, eps, "f64")
        assert np.array_equal(dx, dx64), f"{dt} dx widening"
        assert np.array_equal(orc.bwd_dw(x, dy, eps, dt), orc.bwd_dw(x64, dy64, eps, "f64"))
    # a known bf16 pattern: 0x4040 is 3.0, 0xC080 is -4.0
    xk = np.array([[0x4040, 0xC080]], dtype=np.uint16)
    wk = np.array([0x3F80, 0x3F80], dtype=np.uint16)  # 1.0, 1.0
    y, r = orc.fwd(xk, wk, _eps32(1e-5), "bf16")
    _close(y[0], [3.0 * r[0], -4.0 * r[0]], 1e-15, what="bf16 pattern decode")
    _close(r[0], 1.0 / math.sqrt(12.5 + _eps32(1e-5)), 1e-15, what="bf16 pattern r")


def pin_row_selection(orc):
    """Row-sampled calls return exactly the rows of the full call."""
    rng = np.random.default_rng(31)
    M, N, eps = 9, 17, 1e-5
    x = rng.standard_normal((M, N)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, N).astype(np.float32)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    y, r = orc.fwd(x, w, eps, "f32")
    dx, _ = orc.bwd_dx(x, w, dy, eps, "f32")
    rows = np.array([8, 0, 3])
    ys, rs = orc.fwd(x, w, eps, "f32", rows=rows)
    dxs, rs2 = orc.bwd_dx(x, w, dy, eps, "f32", rows=rows)
    assert np.array_equal(ys, y[rows]) and np.array_equal(rs, r[rows]) and np.array_equal(rs2, r[rows])
    assert np.array_equal(dxs, dx[rows])


ALL_PINS = [
    pin_worked_examples,
    pin_one_column,
    pin_constant_rows,
    pin_zero_cases,
    pin_unit_mean_square,
    pin_scaling,
    pin_finite_differences,
    pin_backward_closed_forms,
    pin_torch_reference,
    pin_storage_widening,
    pin_row_selection,
]
