"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small and ragged shapes compare every element; the full-size synthetic
workloads compare sampled rows of y and dx, every rstd, and every dW column
(the oracle computes those exactly one by one), in the launch configuration
the library chooses by default -- the one the benchmark times.
"""

from __future__ import annotations

import json
import os
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
from parity_util import (DT, FORMATS, check_dw, check_rows, check_rstd, gpu_bwd, gpu_fwd, gpu_fwd_residual,  # noqa: E402
                         oracle_row_blocks,
                         term_rms, to_device, to_host, widen)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hello_gpu_ch13_worked_examples.json")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def full_check(x, w, dy, eps, dtype, cfg_f=None, cfg_b=None):
    y, rstd = gpu_fwd(x, w, eps, dtype, cfg=cfg_f)
    oy, orr = oracle.fwd(x, w, eps, dtype)
    check_rows(y, oy, dtype, "y")
    check_rstd(rstd, orr)
    dx, dw = gpu_bwd(x, w, dy, rstd, dtype, cfg=cfg_b)
    odx, orr = oracle.bwd_dx(x, w, dy, eps, dtype)
    check_rows(dx, odx, dtype, "dx", floor=term_rms(x, w, dy, orr, dtype))
    check_dw(dw, oracle.bwd_dw(x, dy, eps, dtype), dtype)
    return y, rstd, dx, dw


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_worked_examples(dtype):
    """hello-gpu ch. 13, section 13.1 and Figure 13.1, on the GPU."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = si.to_storage(np.array([c["x"]], np.float32), dtype)
        w = si.to_storage(np.array(c["w"], np.float32), dtype)
        eps = si.eps_f32(c["eps"])
        y, rstd = gpu_fwd(x, w, eps, dtype)
        assert abs(rstd[0] - c["r"]) <= c["tol"]
        yw = widen(y, dtype)
        for j, v in c["y"].items():
            # printed to 4 decimals; bf16 adds at most 2^-8 relative
            tol = c["tol"] + (2.0 ** -8 * abs(v) if dtype == "bf16" else 0.0)
            assert abs(yw[0, int(j)] - v) <= tol
        oy, orr = oracle.fwd(x, w, eps, dtype)
        check_rows(y, oy, dtype, "y")
        check_rstd(rstd, orr)


SMALL_SHAPES = [
    (1, 1), (3, 13), (33, 257), (7, 8), (5, 64), (17, 128), (129, 1000), (64, 1024), (31, 4096),
    (19, 5120), (9, 7168), (3, 8192), (2, 32768), (2, 65536), (300, 96), (1000, 16), (257, 40),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,N", SMALL_SHAPES, ids=lambda v: str(v))
def test_parity_small(M, N, dtype):
    _say(f"parity_small M={M} N={N} {dtype}")
    x, w, dy = si.random_case(M, N, dtype, seed=1000 + M * 7 + N, dy_scale=1.0 if dtype == "f32" else 1e-2)
    full_check(x, w, dy, si.eps_f32(1e-5), dtype)


def _instantiated_shapes():
    """Every (lanes_per_row, vecs_per_lane, wg_threads, prefetch) kernel the library builds."""
    out = []
    for pf in (0, 1):
        out += [(lpr, 1, 256, pf) for lpr in (1, 2, 4, 8, 16, 32)]
        for lpr, wgs in ((64, (256, 512, 1024)), (128, (256, 512, 1024)), (256, (256, 512, 1024)),
                         (512, (512, 1024)), (1024, (1024,))):
            out += [(lpr, v, wg, pf) for wg in wgs for v in range(1, 9)]
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_vector_kernel(dtype):
    """Each instantiated vector kernel, forced through *_with_config, on a
    ragged row (last vector slot partly empty), a ragged row count, and a grid
    of 2 so workgroups loop over row blocks (and, with prefetch, load past the
    last block)."""
    epv = 4 if dtype == "f32" else 8
    shapes = _instantiated_shapes()
    assert len(shapes) == 204
    for lpr, vpt, wg, pf in shapes:
        nvec = min(lpr * vpt, max(1, lpr * (vpt - 1) + max(1, lpr // 2 + 1)))  # the last slot is partial
        N = nvec * epv
        M = 3 * (wg // lpr) + 1
        # the non-temporal forward loads on every other kernel (a cache hint only)
        cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=lpr, vecs_per_lane=vpt, wg_threads=wg,
                                prefetch=pf, stream_loads=(vpt + pf) % 2, grid=2)
        x, w, dy = si.random_case(M, N, dtype, seed=lpr * 100 + vpt + wg + pf, dy_scale=1e-2)
        _say(f"kernel lpr={lpr} vpt={vpt} wg={wg} pf={pf} N={N} M={M} {dtype}")
        full_check(x, w, dy, si.eps_f32(1e-6), dtype, cfg_f=cfg, cfg_b=cfg)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scalar_path_forced_and_unaligned(dtype):
    """The scalar kernel forced, on aligned buffers and on unaligned views
    (one element into larger buffers; the ladder gives those the element
    kernels, checked here too)."""
    M, N = 37, 4096
    x, w, dy = si.random_case(M, N, dtype, seed=77, dy_scale=1e-2)
    cfg = rn.rmsnorm_config(vector_path=0, grid=5)
    full_check(x, w, dy, si.eps_f32(1e-5), dtype, cfg_f=cfg, cfg_b=cfg)
    xd = to_device(np.concatenate([x.reshape(-1)[:1], x.reshape(-1)]), dtype)[1:]
    wd = to_device(np.concatenate([w[:1], w]), dtype)[1:]
    oy, orr = oracle.fwd(x, w, si.eps_f32(1e-5), dtype)
    for forced in (None, cfg):
        y = torch.full((M * N + 1,), float("nan"), dtype=xd.dtype, device="cuda")[1:]
        rstd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        if forced is None:
            rn.rmsnorm_fwd(xd, wd, si.eps_f32(1e-5), M, N, DT[dtype], y, rstd)
        else:
            rn.rmsnorm_fwd_with_config(xd, wd, si.eps_f32(1e-5), M, N, DT[dtype], y, rstd, forced)
        torch.cuda.synchronize()
        check_rows(to_host(y, dtype).reshape(M, N), oy, dtype, f"y (unaligned, {'scalar' if forced else 'ladder'})")
        check_rstd(rstd.cpu().numpy(), orr)


def test_backward_with_oracle_rstd():
    """Feeding the backward the oracle's rstd (rounded to fp32) separates
    backward error from forward error."""
    M, N, dtype = 64, 4096, "bf16"
    x, w, dy = si.random_case(M, N, dtype, seed=91, dy_scale=1e-2)
    eps = si.eps_f32(1e-6)
    _, orr = oracle.fwd(x, w, eps, dtype, want_y=False)
    dx, dw = gpu_bwd(x, w, dy, orr.astype(np.float32), dtype)
    odx, orr = oracle.bwd_dx(x, w, dy, eps, dtype)
    check_rows(dx, odx, dtype, "dx", floor=term_rms(x, w, dy, orr, dtype))
    check_dw(dw, oracle.bwd_dw(x, dy, eps, dtype), dtype)


def test_invariants_on_gpu():
    """hello-gpu ch. 13, section 13.4: zero input -> zero output, zero weight ->
    zero output; and zero dy -> zero dx and dW."""
    for dtype in ("f32", "bf16"):
        M, N = 8, 1024
        x, w, dy = si.random_case(M, N, dtype, seed=5)
        x[2] = 0
        y, rstd = gpu_fwd(x, w, si.eps_f32(1e-5), dtype)
        assert np.all(widen(y[2], dtype) == 0.0)
        assert rstd[2] == pytest.approx(1.0 / np.sqrt(si.eps_f32(1e-5)), rel=1e-6)
        y0, _ = gpu_fwd(x, np.zeros_like(w), si.eps_f32(1e-5), dtype)
        assert np.all(widen(y0, dtype) == 0.0)
        dx, dw = gpu_bwd(x, w, np.zeros_like(dy), rstd, dtype)
        assert np.all(widen(dx, dtype) == 0.0) and np.all(dw == 0.0)


def test_large_magnitudes_fp32():
    """Rows near 1e15 (squares ~1e30, still finite in fp32 sums) and tiny rows."""
    M, N, dtype = 6, 4096, "f32"
    x, w, dy = si.random_case(M, N, dtype, seed=8)
    scale = np.array([1e15, 1e-15, 1.0, 1e10, 1e-10, 3.0], np.float32)[:, None]
    x = (x * scale).astype(np.float32)
    full_check(x, w, dy, si.eps_f32(1e-5), dtype)


def test_empty_and_degenerate():
    for dtype in ("f32", "bf16"):
        N = 64
        x = torch.empty((0, N), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
        w = torch.ones(N, dtype=x.dtype, device="cuda")
        rn.rmsnorm_fwd(x, w, 1e-5, 0, N, DT[dtype], x, None)
        dw = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        assert rn.rmsnorm_bwd_workspace_bytes(0, N, DT[dtype]) == 0
        rn.rmsnorm_bwd(x, w, x, None, 0, N, DT[dtype], x, dw, None, 0)
        torch.cuda.synchronize()
        assert torch.all(dw == 0)


def test_error_codes_on_device():
    M, N = 16, 256
    x = torch.randn(M, N, device="cuda")
    w = torch.ones(N, device="cuda")
    dx = torch.empty_like(x)
    dw = torch.empty(N, device="cuda")
    rstd = torch.ones(M, device="cuda")
    need = rn.rmsnorm_bwd_workspace_bytes(M, N, rn.F32)
    ws = torch.empty(need // 4 + 64, device="cuda")
    with pytest.raises(rn.RmsnormError) as e:
        rn.rmsnorm_bwd(x, w, x, rstd, M, N, rn.F32, dx, dw, ws, need - 4)
    assert e.value.status == rn.EWORKSPACE
    with pytest.raises(rn.RmsnormError) as e:
        rn.rmsnorm_bwd(x, w, x, rstd, M, N, rn.F32, dx, dw, ws.data_ptr() + 4, need)
    assert e.value.status == rn.EWORKSPACE
    with pytest.raises(rn.RmsnormError) as e:  # 8 lanes x 1 vector cannot cover 64 fp32 vectors
        rn.rmsnorm_fwd_with_config(x, w, 1e-5, M, N, rn.F32, dx, rstd, rn.rmsnorm_config(
            vector_path=1, lanes_per_row=8, vecs_per_lane=1, grid=1))
    assert e.value.status == rn.ECONFIG


# One shape per backward kernel family the ladder picks (and the forward's
# grids): 512-lane rows with two blocks prefetched, whole-wavefront rows (640
# and 320 lanes), the wide-row kernel, narrow rows several to a wavefront, fp32
# rows of 1024 lanes, fp32 weights (the mid-size and the resident forward
# grids), and the element kernels on 64-lane rows 8 to a CU, 512-lane rows
# with 8-byte accesses and fp32 rows with 2 elements per access.
DETERMINISM_CASES = [("bf16", 4096, 4096), ("bf16", 4096, 5120), ("bf16", 8192, 2560), ("bf16", 256, 32768),
                     ("bf16", 65536, 128), ("f32", 1024, 4096), ("bf16w32", 2048, 8192), ("bf16w32", 8192, 4096),
                     ("bf16", 16384, 300), ("bf16", 4096, 4100), ("f32", 2048, 4098)]


@pytest.mark.parametrize("fmt,M,N", DETERMINISM_CASES, ids=lambda v: str(v))
def test_dw_bit_identical_across_reruns(fmt, M, N):
    """Same input -> same y, rstd, dx and dW bits, 10 reruns, each on fresh
    buffers at other addresses ("RMSNorm backward (almost) without the column
    reduction", section "The problem: summing across rows")."""
    act, wst, _ = FORMATS[fmt]
    x, w, dy = si.random_case(M, N, act, seed=123 + N, dy_scale=1e-2, wdtype=wst)
    eps = si.eps_f32(1e-6)
    _say(f"determinism {fmt} {M}x{N}")
    ref_y, rstd = gpu_fwd(x, w, eps, act)
    ref_dx, ref = gpu_bwd(x, w, dy, rstd, act)
    for i in range(10):
        _pad = torch.empty(1 + i * 4096, device="cuda")  # shift the allocator's addresses
        y, rstd2 = gpu_fwd(x, w, eps, act)
        assert np.array_equal(y.view(np.uint8), ref_y.view(np.uint8)) and \
            np.array_equal(rstd2.view(np.uint32), rstd.view(np.uint32)), \
            f"forward bits differ on rerun {i}"
        dx, dw = gpu_bwd(x, w, dy, rstd, act)
        assert np.array_equal(dw.view(np.uint32), ref.view(np.uint32)), f"dW bits differ on rerun {i}"
        assert np.array_equal(dx.view(np.uint8), ref_dx.view(np.uint8)), f"dx bits differ on rerun {i}"
        del _pad
    check_dw(ref, oracle.bwd_dw(x, dy, eps, act), act)


# the headline workload and the widest-row one, with device-resident inputs
DETERMINISM_WORKLOADS = ["bf16_16384x4096", "bf16_32768x8192_outliers"]


@pytest.mark.parametrize("name", DETERMINISM_WORKLOADS)
def test_bits_identical_across_reruns_at_workload_shapes(name):
    """The benchmark's workloads in the default configuration: 10 reruns of
    forward and backward, each writing freshly allocated outputs at other
    addresses, give the same y, rstd, dx and dW bits ("RMSNorm backward
    (almost) without the column reduction", section "The problem: summing
    across rows"). Compared on the device."""
    wl = si.WORKLOADS[name]
    code = DT[wl.dtype]
    x, w, dy = si.make_inputs(wl)
    eps = si.eps_f32(wl.eps)
    M, N = wl.M, wl.N
    xd, wd, dyd = to_device(x, wl.dtype), to_device(w), to_device(dy, wl.dtype)
    nbytes = rn.rmsnorm_bwd_workspace_bytes(M, N, code)

    def run():
        y = torch.empty_like(xd)
        rstd = torch.empty(M, device="cuda")
        rn.rmsnorm_fwd(xd, wd, eps, M, N, code, y, rstd)
        dx = torch.empty_like(xd)
        dw = torch.empty(N, device="cuda")
        ws = torch.full((nbytes // 4 + 64,), float("nan"), device="cuda")
        rn.rmsnorm_bwd(xd, wd, dyd, rstd, M, N, code, dx, dw, ws, nbytes)
        torch.cuda.synchronize()
        return y.view(torch.int16), rstd.view(torch.int32), dx.view(torch.int16), dw.view(torch.int32)

    _say(f"determinism at {name}")
    ref = run()
    for i in range(10):
        _pad = torch.empty(1 + i * 65536, device="cuda")  # shift the allocator's addresses
        out = run()
        for what, a, b in zip(("y", "rstd", "dx", "dW"), out, ref):
            assert torch.equal(a, b), f"{what} bits differ on rerun {i}"
        del out, _pad
    check_dw(ref[3].view(torch.float32).cpu().numpy(), oracle.bwd_dw(x, dy, eps, wl.dtype), wl.dtype)


@pytest.mark.parametrize("name", ["bf16_16384x4096", "bf16_32768x8192_outliers", "bf16_16384x4100",
                                  "bf16_qknorm_1048576x128"])
def test_dw_plain_relative_bound_at_workloads(name):
    """dW of the default backward against the oracle under the plain relative
    bound |g - o| <= 1e-3 |o_j| on every column, with no floor, at the
    workloads where it holds: their row kernels (the LDS-staged kernel, the
    register kernel with two blocks prefetched or on 256-lane workgroups, the
    element kernel) keep fp32 block sums folded into fp64 totals and the
    combine adds the partial rows in fp64, so a column whose total nearly
    cancels keeps mostly the fp32 partial rows' and rstd's rounding (at bf16
    16384x4096 the smallest |dW_j| is 5.3e-5). With plain fp32 running sums
    the first three had 2, 2 and 0 such columns above the bound (max relative
    error 5.2e-3, 1.3e-3, 9.7e-4)."""
    wl = si.workload(name)
    _say(f"plain dW bound: {name}")
    x, w, dy = si.make_inputs(wl)
    eps = si.eps_f32(wl.eps)
    _, rstd = gpu_fwd(x, w, eps, wl.dtype)
    _, dw = gpu_bwd(x, w, dy, rstd, wl.dtype)
    o = oracle.bwd_dw(x, dy, eps, wl.dtype)
    err = np.abs(dw.astype(np.float64) - o)
    rel = err / np.abs(o)
    worst = int(np.argmax(rel))
    assert rel.max() <= 1e-3, f"{name}: column {worst}: dW {dw[worst]!r} oracle {o[worst]!r} rel {rel.max():.3e}"


def _sample_rows(M, k=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(k, M), replace=False).tolist())
    rows |= {0, 1, M - 2, M - 1}
    return np.array(sorted(r for r in rows if 0 <= r < M), dtype=np.int64)


@pytest.mark.parametrize("name", list(si.WORKLOADS))
def test_full_size_workload(name):
    """Full-size synthetic workload in the default launch configuration (the
    one the benchmark times): every row of y and dx, streamed through the
    oracle in blocks of rows, every rstd and every dW column."""
    wl = si.WORKLOADS[name]
    _say(f"workload {name}: generating inputs")
    x, w, dy = si.make_inputs(wl)
    eps = si.eps_f32(wl.eps)
    _say(f"workload {name}: gpu")
    y, rstd = gpu_fwd(x, w, eps, wl.dtype)
    dx, dw = gpu_bwd(x, w, dy, rstd, wl.dtype)
    _say(f"workload {name}: oracle, every row")
    worst = {"y": 0.0, "dx": 0.0}
    orr = np.empty(wl.M)
    for rows, oy, r, odx in oracle_row_blocks(x, w, dy, eps, wl.dtype):
        orr[rows] = r
        worst["y"] = max(worst["y"], check_rows(y[rows], oy, wl.dtype, "y")["max_gate_ratio"])
        idx = np.arange(rows.start, rows.stop)
        worst["dx"] = max(worst["dx"], check_rows(dx[rows], odx, wl.dtype, "dx",
                                                  floor=term_rms(x, w, dy, r, wl.dtype, rows=idx))["max_gate_ratio"])
    check_rstd(rstd, orr)
    d = check_dw(dw, oracle.bwd_dw(x, dy, eps, wl.dtype), wl.dtype)
    _say(f"workload {name}: {wl.M} rows; worst err/bound y {worst['y']:.3f}, dx {worst['dx']:.3f}; dW max rel err "
         f"{d['max_rel_err']:.2e}, {d['cols_above_plain_rel_tol']} of {d['cols']} columns above the plain relative "
         f"bound (gate: {d['gate']})")
    assert np.all(np.isfinite(widen(y, wl.dtype))) and np.all(np.isfinite(widen(dx, wl.dtype)))


def test_beyond_4gib_tensors():
    """bf16 1048576 x 2560: 2.7e9 elements, 5.4 GB per tensor, so element
    indices pass 2^31 and byte offsets pass 2^32. Inputs are drawn on the
    device (seeded); sampled rows, including the last ones, go to the host for
    the oracle. dW is checked column by column against the fp64 sum of
    dy * x * r over all rows, with r = 1/sqrt(mean(x^2) + eps) also in fp64
    (plain PyTorch, in row chunks): no part of that reference comes from the
    kernels' outputs."""
    M, N, dtype = 1 << 20, 2560, "bf16"
    eps = si.eps_f32(1e-6)
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    _say("4 GiB+: generating on the device")
    x = torch.randn((M, N), generator=g, device="cuda").to(torch.bfloat16)
    dy = (torch.randn((M, N), generator=g, device="cuda") * 1e-2).to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn(N, generator=g, device="cuda")).to(torch.bfloat16)
    y = torch.empty_like(x)
    rstd = torch.empty(M, device="cuda")
    _say("4 GiB+: forward")
    rn.rmsnorm_fwd(x, w, eps, M, N, rn.BF16, y, rstd)
    dx = torch.empty_like(x)
    dw = torch.empty(N, device="cuda")
    nbytes = rn.rmsnorm_bwd_workspace_bytes(M, N, rn.BF16)
    ws = torch.empty(nbytes // 4 + 64, device="cuda")
    _say("4 GiB+: backward")
    rn.rmsnorm_bwd(x, w, dy, rstd, M, N, rn.BF16, dx, dw, ws, nbytes)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([_sample_rows(M, k=24, seed=7), np.arange(M - 8, M)])).astype(np.int64)
    ri = torch.from_numpy(rows).cuda()
    xs, dys = to_host(x[ri], dtype), to_host(dy[ri], dtype)
    wh = to_host(w, dtype)
    oy, orr = oracle.fwd(xs, wh, eps, dtype)
    check_rows(to_host(y[ri], dtype), oy, dtype, "y (rows past 4 GiB)")
    check_rstd(rstd[ri].cpu().numpy(), orr)
    odx, orr = oracle.bwd_dx(xs, wh, dys, eps, dtype)
    check_rows(to_host(dx[ri], dtype), odx, dtype, "dx (rows past 4 GiB)", floor=term_rms(xs, wh, dys, orr, dtype))
    _say("4 GiB+: dW reference")
    ref = torch.zeros(N, dtype=torch.float64, device="cuda")
    for s in range(0, M, 1 << 16):
        e = min(M, s + (1 << 16))
        xd = x[s:e].double()
        r = 1.0 / torch.sqrt((xd * xd).mean(dim=1) + float(eps))
        ref += (dy[s:e].double() * xd * r[:, None]).sum(0)
        del xd
    ref = ref.cpu().numpy()
    err = np.abs(dw.cpu().numpy().astype(np.float64) - ref)
    bound = 1e-3 * np.maximum(np.abs(ref), 1e-2 * np.sqrt(np.mean(ref * ref)))
    assert np.all(err <= bound), f"dW: max err {err.max()}"
    del x, dy, y, dx, ws
    torch.cuda.empty_cache()


DEEP_SHAPES = [(1, 256), (2, 256), (4, 256), (8, 256), (16, 256), (32, 256), (64, 1024), (128, 1024),
               (256, 1024), (512, 512), (1024, 1024)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_deep_prefetch_kernel(dtype):
    """The backward kernels with two row blocks prefetched, forced through
    *_with_config: a ragged row, 6 row blocks over a grid of 2, so each
    workgroup walks 3 blocks (both ring slots, and the exit after the first)."""
    epv = 4 if dtype == "f32" else 8
    for lpr, wg in DEEP_SHAPES:
        nvec = max(1, lpr // 2 + 1) if lpr > 1 else 1
        N = nvec * epv
        M = 5 * (wg // lpr) + 1
        cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=lpr, vecs_per_lane=1, wg_threads=wg, prefetch=2,
                                grid=2)
        x, w, dy = si.random_case(M, N, dtype, seed=lpr * 31 + wg, dy_scale=1e-2)
        _say(f"deep prefetch lpr={lpr} wg={wg} N={N} M={M} {dtype}")
        full_check(x, w, dy, si.eps_f32(1e-6), dtype, cfg_b=cfg)


# Backward rows of 257..1024 vectors on whole wavefronts that are not a power
# of two: the kernels whose row is the whole workgroup, sized at launch.
ROWWG_LANES = (320, 384, 448, 576, 640, 704, 832, 896, 960)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_workgroup_row_kernel(dtype):
    """Workgroup-sized backward rows at every prefetch depth, forced through
    *_with_config: the last wavefront partly empty, 7 rows over grids of 2 and
    3 (workgroups walk 2 to 4 rows: both ring slots and the early exit); the
    ladder's own choice at the same width as well."""
    epv = 4 if dtype == "f32" else 8
    for lanes in ROWWG_LANES:
        nvec = lanes - 37
        N, M = nvec * epv, 7
        x, w, dy = si.random_case(M, N, dtype, seed=lanes * 3 + 1, dy_scale=1e-2)
        for pf in (1, 2):
            for grid in (2, 3):
                cfg = rn.rmsnorm_config(vector_path=1, lanes_per_row=lanes, vecs_per_lane=1, wg_threads=lanes,
                                        prefetch=pf, grid=grid)
                _say(f"workgroup row lanes={lanes} pf={pf} grid={grid} N={N} M={M} {dtype}")
                full_check(x, w, dy, si.eps_f32(1e-6), dtype, cfg_b=cfg)
        _say(f"workgroup row width, the ladder's own choice: N={N} {dtype}")
        full_check(x, w, dy, si.eps_f32(1e-6), dtype)


@pytest.mark.parametrize("dtype,M,N", [("bf16", 1, 4096), ("bf16", 16, 128), ("f32", 1, 1024), ("bf16", 1, 32768),
                                       ("bf16", 8, 1024), ("bf16", 2, 4096), ("bf16", 4, 4096), ("f32", 4, 4096),
                                       ("bf16", 8, 2048), ("bf16", 4, 2560)], ids=lambda v: str(v))
def test_single_workgroup_backward_writes_dw(dtype, M, N):
    """A backward whose row kernel runs as one workgroup writes dW itself (no
    combine launch), including walks of 2 to 4 row blocks (the depth-2
    prefetch kernel at 4 x 4096, 256-lane rows at 8 x 2048, whole-wavefront
    rows at 4 x 2560): dW and dx against the oracle, equal to the two-call
    path (rows, then combine, through the workspace), nothing written around a
    16-byte aligned dW inside a larger buffer, and, with dW not 16-byte
    aligned, the combine path again."""
    x, w, dy = si.random_case(M, N, dtype, seed=M * 31 + N, dy_scale=1e-2)
    eps = si.eps_f32(1e-6)
    code = DT[dtype]
    assert rn.rmsnorm_query_config(M, N, code, 1).grid == 1
    _say(f"single-workgroup backward {dtype} {M}x{N}")
    _, rstd = gpu_fwd(x, w, eps, dtype)
    dx, dw = gpu_bwd(x, w, dy, rstd, dtype)
    odx, orr = oracle.bwd_dx(x, w, dy, eps, dtype)
    check_rows(dx, odx, dtype, "dx", floor=term_rms(x, w, dy, orr, dtype))
    check_dw(dw, oracle.bwd_dw(x, dy, eps, dtype), dtype)
    # the two-call path through the workspace
    xd, wd, gd = to_device(x, dtype), to_device(w), to_device(dy, dtype)
    rd = torch.from_numpy(rstd).cuda()
    dxd = torch.empty_like(xd)
    nb = rn.rmsnorm_bwd_workspace_bytes(M, N, code)
    ws = torch.empty(nb // 4 + 64, device="cuda")
    P = rn.rmsnorm_bwd_rows(xd, wd, gd, rd, M, N, code, dxd, ws, nb)
    dw2 = torch.full((N,), float("nan"), device="cuda")
    rn.rmsnorm_bwd_combine(ws, P, N, dw2)
    torch.cuda.synchronize()
    assert P == 1 and np.array_equal(dw2.cpu().numpy(), dw), "two-call dW differs"
    # dW one float past a 16-byte boundary: the combine path
    big = torch.full((N + 4,), float("nan"), device="cuda")
    dw3 = big[1:N + 1]
    rn.rmsnorm_bwd(xd, wd, gd, rd, M, N, code, dxd, dw3, ws, nb)
    torch.cuda.synchronize()
    assert np.array_equal(dw3.cpu().numpy(), dw), "dW through the combine differs"
    assert torch.isnan(big[0]) and torch.isnan(big[N + 1:]).all(), "wrote outside dW"
    # dW 16 bytes into a larger buffer: the direct write, and nothing around it
    big = torch.full((N + 8,), float("nan"), device="cuda")
    dw4 = big[4:N + 4]
    rn.rmsnorm_bwd(xd, wd, gd, rd, M, N, code, dxd, dw4, ws, nb)
    torch.cuda.synchronize()
    assert np.array_equal(dw4.cpu().numpy(), dw), "direct dW differs"
    assert torch.isnan(big[:4]).all() and torch.isnan(big[N + 4:]).all(), "the direct write went outside dW"


def test_single_workgroup_residual_backward():
    """The fused residual backward on one workgroup (2 rows of 4096) writes dW
    itself: dx and dW against the oracle's residual reading."""
    M, N = 2, 4096
    code = rn.BF16
    assert rn.rmsnorm_query_config(M, N, code, 1).grid == 1
    x, w, dy = si.random_case(M, N, "bf16", seed=77, dy_scale=1e-2)
    res = si.random_tensor((M, N), "bf16", seed=78)
    dh = si.random_tensor((M, N), "bf16", seed=79, scale=1e-2)
    eps = si.eps_f32(1e-6)
    h, _, rstd = gpu_fwd_residual(x, res, w, eps, "bf16")
    dx, dw = gpu_bwd(h, w, dy, rstd, "bf16", dh=dh)
    odx, orr = oracle.bwd_dx(x, w, dy, eps, "bf16", res=res, dh=dh)
    check_rows(dx, odx, "bf16", "dx", floor=term_rms(h, w, dy, orr, "bf16", dh=dh))
    check_dw(dw, oracle.bwd_dw(x, dy, eps, "bf16", res=res), "bf16")


def test_element_rows_keep_the_combine_for_few_rows():
    """The single-workgroup rule was measured on the vector kernels only; rows
    that are not a multiple of 16 bytes (the element kernels) keep their grid
    and the combine at a few rows, and match the oracle."""
    for dtype, M, N in (("bf16", 3, 5001), ("f32", 1, 257)):
        code = DT[dtype]
        c = rn.rmsnorm_query_config(M, N, code, 1)
        assert c.vector_path == 3 and c.grid == M, (dtype, M, N, c.as_dict())
        x, w, dy = si.random_case(M, N, dtype, seed=N, dy_scale=1e-2)
        eps = si.eps_f32(1e-6)
        _, rstd = gpu_fwd(x, w, eps, dtype)
        dx, dw = gpu_bwd(x, w, dy, rstd, dtype)
        odx, orr = oracle.bwd_dx(x, w, dy, eps, dtype)
        check_rows(dx, odx, dtype, "dx", floor=term_rms(x, w, dy, orr, dtype))
        check_dw(dw, oracle.bwd_dw(x, dy, eps, dtype), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scalar_backward_sums_in_lds_and_in_memory(dtype):
    """The scalar backward keeps its dW running sums in LDS up to 16384
    columns and in its partial row in memory beyond: both sides of that limit,
    forced through the scalar path with a grid that makes workgroups walk
    several rows, against the oracle."""
    for N in (16384, 16385):
        M = 37
        x, w, dy = si.random_case(M, N, dtype, seed=N + 5, dy_scale=1e-2)
        cfg = rn.rmsnorm_config(vector_path=0, grid=5)
        _say(f"scalar backward N={N} {dtype}")
        full_check(x, w, dy, si.eps_f32(1e-6), dtype, cfg_f=cfg, cfg_b=cfg)
