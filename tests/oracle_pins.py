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
    implementation of the same definition,
  * library conversions for the storage formats: numpy's float16 decode of
    every bit pattern, numpy's float64 -> float16/float32 casts and torch's
    float32 -> bfloat16 cast for round-to-nearest-even, plus hand-derived ties,
  * for the fused residual add (the profiling page, Problem 15): the worked
    example reached as x + res, exact rounding cases of the stored sum, and
    central finite differences of L = sum(dy * y(x + res)) + sum(dh * (x + res)).

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


def pin_fp16_decode(orc):
    """Every finite fp16 bit pattern decodes to numpy's float16 value. (The
    residual forward with res = 0 returns the stored sum x + 0 = x.)"""
    bits = np.arange(1 << 16, dtype=np.uint16)
    vals = bits.view(np.float16)
    keep = np.isfinite(vals)
    x = vals[keep].reshape(1, -1)
    h, _, _ = orc.fwd_residual(x, np.zeros_like(x), np.ones(x.shape[1], np.float16), 1.0, "f16", want_y=False)
    assert np.array_equal(h[0], x[0].astype(np.float64)), "fp16 decode differs from numpy"


def pin_rounding(orc):
    """Round to nearest, ties to even, against library conversions: numpy's
    float64 -> float16 and float64 -> float32 casts, torch's float32 -> bfloat16
    cast (on float32-exact inputs); plus hand-derived ties and overflow."""
    import torch

    rng = np.random.default_rng(37)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000),
                        rng.standard_normal(500) * 1e-6, [0.0, -0.0, 65504.0, 65519.9, -70000.0, 6e-8, 3e-8]])
    got16 = orc.round(v, "f16")
    with np.errstate(over="ignore"):
        want16 = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(got16, want16), "fp16 rounding differs from numpy"
    got32 = orc.round(v, "f32")
    assert np.array_equal(got32, v.astype(np.float32).astype(np.float64)), "fp32 rounding differs"
    v32 = v.astype(np.float32).astype(np.float64)
    gotb = orc.round(v32, "bf16")
    wantb = torch.tensor(v32, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(gotb, wantb), "bf16 rounding differs from torch"
    # ties: bf16 keeps 8 significant bits, so 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -9 + 2 ** -17])
    assert np.array_equal(orc.round(ties, "bf16"), [1.0, 1 + 2 ** -6, -1.0, 2 ** -9])
    assert np.array_equal(orc.round(np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 65520.0]), "f16"),
                          [1.0, 1 + 2 ** -9, np.inf])


def pin_residual_worked_example(orc):
    """hello-gpu ch. 13, Figure 13.1, reached through the residual form:
    x + res = [3, 4, -3, -4] (exact) must give the printed r and y."""
    with open(GOLDEN) as f:
        c = json.load(f)["cases"][1]
    x = _f32([[1.0, 2.0, -1.0, -2.0]])
    res = _f32([[2.0, 2.0, -2.0, -2.0]])
    h, y, r = orc.fwd_residual(x, res, _f32(c["w"]), _eps32(c["eps"]), "f32")
    assert np.array_equal(h[0], c["x"]), "residual sum"
    assert abs(r[0] - c["r"]) <= c["tol"]
    for j, v in c["y"].items():
        assert abs(y[0, int(j)] - v) <= c["tol"]


def pin_residual_rounding(orc):
    """The stored sum is rounded to the activation format before it is
    normalised: bf16 1 + 2^-8 is a tie and stays 1; 1 + 3*2^-8 goes to 1 + 2^-6.
    With res = 0 the forward and backward equal the plain ones exactly."""
    bf = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    x = bf([[1.0, 1.0, 2.0, -3.0]])
    res = bf([[2 ** -8, 3 * 2 ** -8, 0.0, 0.0]])
    w = bf([1.0, 1.0, 1.0, 1.0])
    h, y, r = orc.fwd_residual(x, res, w, 0.0, "bf16")
    assert np.array_equal(h[0], [1.0, 1 + 2 ** -6, 2.0, -3.0]), h
    ms = np.mean(h[0] ** 2)
    _close(r[0], 1 / np.sqrt(ms), 1e-15, what="r of the stored sum")
    rng = np.random.default_rng(41)
    xb = bf(rng.standard_normal((3, 16)))
    wb = bf(rng.uniform(0.5, 1.5, 16))
    dyb = bf(rng.standard_normal((3, 16)))
    zero = np.zeros_like(xb)
    h0, y0, r0 = orc.fwd_residual(xb, zero, wb, 1e-5, "bf16")
    y1, r1 = orc.fwd(xb, wb, 1e-5, "bf16")
    assert np.array_equal(y0, y1) and np.array_equal(r0, r1)
    dx0, _ = orc.bwd_dx(xb, wb, dyb, 1e-5, "bf16", res=zero, dh=zero)
    dx1, _ = orc.bwd_dx(xb, wb, dyb, 1e-5, "bf16")
    assert np.array_equal(dx0, dx1)
    assert np.array_equal(orc.bwd_dw(xb, dyb, 1e-5, "bf16", res=zero), orc.bwd_dw(xb, dyb, 1e-5, "bf16"))


def pin_residual_finite_differences(orc):
    """L = sum(dy * y(x + res)) + sum(dh * (x + res)): central differences in x
    and in res both equal the residual backward's dx (fp64 storage, where the
    stored sum is exact); its dW equals the plain dW at h = x + res."""
    rng = np.random.default_rng(43)
    M, N, eps = 3, 6, 1e-3
    x = rng.standard_normal((M, N))
    res = rng.standard_normal((M, N))
    w = rng.uniform(0.5, 1.5, N)
    dy = rng.standard_normal((M, N))
    dh = rng.standard_normal((M, N))

    def loss(xx, rr):
        h, y, _ = orc.fwd_residual(xx, rr, w, eps, "f64")
        return float(np.sum(dy * y) + np.sum(dh * h))

    dx, _ = orc.bwd_dx(x, w, dy, eps, "f64", res=res, dh=dh)
    for which in ("x", "res"):
        fd = np.empty_like(x)
        for i in range(M):
            for j in range(N):
                hstep = 1e-6 * max(1.0, abs(x[i, j]))
                a, b = x.copy(), x.copy()
                ra, rb = res.copy(), res.copy()
                if which == "x":
                    a[i, j] += hstep
                    b[i, j] -= hstep
                else:
                    ra[i, j] += hstep
                    rb[i, j] -= hstep
                fd[i, j] = (loss(a, ra) - loss(b, rb)) / (2 * hstep)
        _close(dx, fd, 0.0, atol=1e-7 * max(1.0, np.max(np.abs(fd))), what=f"residual dx vs d/d{which}")
    _close(orc.bwd_dw(x, dy, eps, "f64", res=res), orc.bwd_dw(x + res, dy, eps, "f64"), 1e-13, atol=1e-15,
           what="residual dW")


def pin_weight_dtype(orc):
    """Weights in their own format widen exactly: bf16 or fp16 activations with
    fp32 weights equal the same numbers given as fp64 weights."""
    rng = np.random.default_rng(47)
    for dt, mk in (("bf16", lambda a: (np.asarray(a, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)),
                   ("f16", lambda a: np.asarray(a, np.float16))):
        x = mk(rng.standard_normal((3, 20)))
        dy = mk(rng.standard_normal((3, 20)))
        w32 = rng.uniform(0.5, 1.5, 20).astype(np.float32)
        y_a, r_a = orc.fwd(x, w32, 1e-5, dt, wdtype="f32")
        y_b, r_b = orc.fwd(x, w32.astype(np.float64), 1e-5, dt, wdtype="f64")
        assert np.array_equal(y_a, y_b) and np.array_equal(r_a, r_b)
        d_a, _ = orc.bwd_dx(x, w32, dy, 1e-5, dt, wdtype="f32")
        d_b, _ = orc.bwd_dx(x, w32.astype(np.float64), dy, 1e-5, dt, wdtype="f64")
        assert np.array_equal(d_a, d_b)
        y_c, _ = orc.fwd(x, w32, 1e-5, dt, wdtype="f32")
        assert not np.array_equal(y_c, orc.fwd(x, np.ones(20, np.float32), 1e-5, dt, wdtype="f32")[0])


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
    pin_fp16_decode,
    pin_rounding,
    pin_residual_worked_example,
    pin_residual_rounding,
    pin_residual_finite_differences,
    pin_weight_dtype,
]
