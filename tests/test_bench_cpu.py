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
