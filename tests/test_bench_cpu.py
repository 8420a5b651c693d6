"""Host logic of bench.py that needs no GPU: the counter-traffic lookup and its
keys, the idle-check parsing, and the one-GPU refusal."""

import importlib.util
import json
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


CFG = {"vector_path": 1, "lanes_per_row": 512, "vecs_per_lane": 1, "wg_threads": 512, "rows_per_wg": 1,
       "prefetch": 2, "stream_loads": 0, "grid": 256, "partial_rows": 256, "partial_stride": 4096}


def test_launch_key(bench):
    assert bench.launch_key(CFG) == [1, 512, 1, 512, 2, 0, 256]
    loop = dict(CFG, vector_path=5, lanes_per_row=1024, vecs_per_lane=4, wg_threads=1024, prefetch=0, grid=64,
                kept_vecs=16)
    assert bench.launch_key(loop) == [5, 1024, 4, 1024, 0, 0, 64, 16]


def test_row_kernel_name(bench):
    base = dict(vector_path=1, copy_mode=0)
    assert bench.row_kernel_name(base) == "bwd_vec"
    assert bench.row_kernel_name(dict(base, copy_mode=1)) == "bwd_lds"
    assert bench.row_kernel_name(dict(vector_path=2, copy_mode=0)) == "bwd_wide"
    assert bench.row_kernel_name(dict(vector_path=2, copy_mode=1)) == "bwd_wide_lds"
    assert bench.row_kernel_name(dict(vector_path=3, copy_mode=0)) == "bwd_elem"
    assert bench.row_kernel_name(dict(vector_path=4, copy_mode=0)) == "bwd_split"
    assert bench.row_kernel_name(dict(vector_path=0, copy_mode=0)) == "bwd_scalar"


def test_source_hash_covers_kernels_not_the_host_ladder(bench, tmp_path, monkeypatch):
    """Counters stay valid across host-only changes (the ladder, the launches)
    and not across kernel changes."""
    csrc = tmp_path / "memory_bound_normalization_rmsnorm_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "memory_bound_normalization_rmsnorm_amd", "csrc"), csrc)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash()
    assert len(h0) == 16 and h0 == bench.source_hash()
    with open(csrc / "rmsn_api.cpp", "a") as f:
        f.write("\n// host-only change\n")
    assert bench.source_hash() == h0
    with open(csrc / "rmsn_bwd_kernels.h", "a") as f:
        f.write("\n// kernel change\n")
    assert bench.source_hash() != h0


def test_load_traffic_needs_same_sources_and_launch(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("abc", "bwd_rows", "w", [1]) is None          # no file
    (tmp_path / "profiles").mkdir()
    entry = {"source_hash": "abc", "launch": bench.launch_key(CFG), "traffic_bytes_per_launch": 407498086}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"bwd_rows:wl": entry}))
    key = bench.launch_key(CFG)
    assert bench.load_traffic("abc", "bwd_rows", "wl", key) == 407498086
    assert bench.load_traffic("abd", "bwd_rows", "wl", key) is None         # other kernel sources
    assert bench.load_traffic("abc", "bwd_rows", "wl", key[:-1] + [512]) is None  # other grid
    assert bench.load_traffic("abc", "fwd", "wl", key) is None              # other kernel
    (tmp_path / "profiles" / "traffic.json").write_text("{ not json")
    assert bench.load_traffic("abc", "bwd_rows", "wl", key) is None


def test_idle_check_parsing(bench):
    doc = {"gpu_data": [{"gpu": 0, "usage": {"gfx_activity": {"value": 3, "unit": "%"},
                                             "umc_activity": {"value": 1, "unit": "%"}},
                         "mem_usage": {"total_vram": {"value": 294896, "unit": "MB"},
                                       "used_vram": {"value": 283, "unit": "MB"}}}]}
    assert bench._find(doc, "umc_activity") == {"value": 1, "unit": "%"}
    assert bench._find(doc, "missing") is None
    assert bench.smi_brief(None) is None
    assert bench.smi_brief({"tool": "amd-smi", "gfx_activity": 3, "raw": "..."}) == {
        "tool": "amd-smi", "gfx_activity": 3, "umc_activity": None, "used_vram": None, "total_vram": None}


def test_more_than_one_gpu_is_refused(bench, capsys):
    assert bench.main(["--gpus", "2"]) == 2
    out = json.loads(capsys.readouterr().out.strip())
    assert "one GPU only" in out["error"]


def test_graph_launches_independent_of_steps(bench):
    # about 50 ms per replay, at least 200 launches, at most 4000
    assert bench.graph_launches(402_743_296) == 745        # backward rows at bf16 16384 x 4096 (~67 us)
    assert bench.graph_launches(268_509_184) == 1118
    assert bench.graph_launches(16_384) == bench.GRAPH_MAX_LAUNCHES   # a few-us kernel
    assert bench.graph_launches(10 << 30) == bench.GRAPH_MIN_LAUNCHES


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_threaded_oracle_pass_matches_the_plain_oracle(bench, threads):
    """The all-cores CPU baseline runs the oracle on row blocks in threads and
    adds the per-block dW in block order: the same y, r and dx as one call,
    and dW equal to the sequential sum up to fp64 rounding."""
    import numpy as np

    import oracle
    import synthetic_inputs as si

    x, w, dy = si.random_case(37, 96, "bf16", seed=11, dy_scale=1e-2)
    eps = si.eps_f32(1e-6)
    y, r, dx, dw = bench.oracle_pass(x, w, dy, eps, "bf16", threads, keep=True)
    oy, orr = oracle.fwd(x, w, eps, "bf16")
    odx, _ = oracle.bwd_dx(x, w, dy, eps, "bf16")
    odw = oracle.bwd_dw(x, dy, eps, "bf16")
    assert np.array_equal(y, oy) and np.array_equal(r, orr) and np.array_equal(dx, odx)
    assert np.allclose(dw, odw, rtol=1e-13, atol=1e-15)
    _, r2, dx2, dw2 = bench.oracle_pass(x, w, dy, eps, "bf16", threads, keep=False)
    assert dx2 is None and np.array_equal(r2, orr) and np.array_equal(dw2, dw)


def test_validate_checks_every_row(bench):
    """validate() gates every row of y and dx (in blocks), every rstd and every
    dW column: the oracle's own values rounded to bf16 pass, and one wrong
    element in the last row fails."""
    import types

    import numpy as np

    import synthetic_inputs as si

    M, N = 300, 64
    x, w, dy = si.random_case(M, N, "bf16", seed=12, dy_scale=1e-2)
    eps = si.eps_f32(1e-6)
    y, r, dx, dw = bench.oracle_pass(x, w, dy, eps, "bf16", 4, keep=True)
    wl = types.SimpleNamespace(M=M, N=N, dtype="bf16")
    gpu = (si.to_storage(y.astype(np.float32), "bf16"), r.astype(np.float32),
           si.to_storage(dx.astype(np.float32), "bf16"), dw.astype(np.float32))
    ref = {"y": y, "rstd": r, "dx": dx, "dw": dw}
    stats = bench.validate(wl, gpu, ref, (x, w, dy), block=64)
    assert stats["passed"] and stats["rows_checked"] == M
    assert stats["dw_cols_above_plain_rel_tol"] == 0 and stats["y_max_gate_ratio"] <= 1.0
    bad = gpu[2].copy()
    bad[M - 1, N - 1] ^= np.uint16(0x4000)  # a large change to one dx element of the last row
    with pytest.raises(AssertionError):
        bench.validate(wl, (gpu[0], gpu[1], bad, gpu[3]), ref, (x, w, dy), block=64)


@pytest.mark.parametrize("variant,fmt", [("fused", "bf16"), ("fused", "bf16w32"), ("residual", "f16"),
                                         ("residual_unfused", "bf16")])
def test_cell_check_against_the_oracle(bench, variant, fmt):
    """The cells-mode gate: outputs equal to the oracle's values rounded once to
    storage pass; one wrong dx element in a sampled row fails."""
    import numpy as np
    import torch

    import oracle
    from parity_util import to_host

    M, N = 70, 48
    act, es, wsz = bench.FMT[fmt]
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[act]
    g = torch.Generator().manual_seed(5)
    base = {"x": torch.randn((M, N), generator=g).to(tdt), "dy": (torch.randn((M, N), generator=g) * 1e-2).to(tdt)}
    resid = variant.startswith("residual")
    if resid:
        base["res"] = torch.randn((M, N), generator=g).to(tdt)
        base["dh"] = (torch.randn((M, N), generator=g) * 1e-2).to(tdt)
    wdt = "f32" if wsz == 4 else act
    w = (1 + 0.1 * torch.randn(N, generator=g)).to(torch.float32 if wsz == 4 else tdt)
    eps = float(np.float32(1e-6))
    ref = bench.cell_reference(base, w, eps, act, wdt, M, N, to_host)
    assert ref["rows"][0] == 0 and ref["rows"][-1] == M - 1
    xh, dyh = to_host(base["x"], act), to_host(base["dy"], act)
    res = to_host(base["res"], act) if resid else None
    dh = to_host(base["dh"], act) if resid else None
    wh = to_host(w, wdt)
    if resid:
        h, y, r = oracle.fwd_residual(xh, res, wh, eps, act, wdtype=wdt)
    else:
        (y, r), h = oracle.fwd(xh, wh, eps, act, wdtype=wdt), None
    dx, _ = oracle.bwd_dx(xh, wh, dyh, eps, act, res=res, dh=dh, wdtype=wdt)
    s = {"y": torch.from_numpy(y).to(tdt), "dx": torch.from_numpy(dx).to(tdt),
         "rstd": torch.from_numpy(r.astype(np.float32))}
    if resid:
        s["h"] = torch.from_numpy(h).to(tdt)
    dw = torch.from_numpy(oracle.bwd_dw(xh, dyh, eps, act, res=res).astype(np.float32))
    out = bench.cell_check(s, dw, ref, act, variant, resid, to_host)
    assert out["passed"] and out["rows_checked"] == min(M, bench.CELL_PARITY_ROWS)
    k = int(ref["rows"][3])
    s["dx"][k, 5] = s["dx"][k, 5] * 3 + 1
    with pytest.raises(AssertionError):
        bench.cell_check(s, dw, ref, act, variant, resid, to_host)
