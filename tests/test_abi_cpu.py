"""The C-ABI library on a machine without a GPU: it loads, exports every
symbol the headers declare, and rejects bad arguments before any HIP call.
The ladder (a pure host function) picks the documented shapes."""

import os
import re

import pytest

import memory_bound_normalization_rmsnorm_amd as rn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions(headers=None):
    names = set()
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h") and (headers is None or h in headers):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(rmsn\w*)\s*\(", src))
    return sorted(names)


def test_exports_every_declared_symbol():
    """The product library exports every function include/rmsnorm.h declares
    and no measurement code; the measurement library exports the probes and
    the unfused reference kernels."""
    names = declared_functions({"rmsnorm.h"})
    assert "rmsnorm_fwd" in names and "rmsnorm_bwd" in names
    for n in names:
        assert hasattr(rn.lib, n), f"{n} declared but not exported"
    assert set(names) == set(rn.EXPORTED)
    bench = declared_functions({"rmsnorm_probe.h", "rmsnorm_baseline.h"})
    assert set(bench) == set(rn.BENCH_EXPORTED)
    for n in bench:
        assert hasattr(rn.bench_lib(), n), f"{n} declared but not exported by the measurement library"
        with pytest.raises(AttributeError):
            getattr(rn.lib, n)
    assert set(declared_functions()) == set(names) | set(bench)


def test_build_info_and_status_strings():
    assert "gfx950" in rn.rmsnorm_build_info()
    assert rn.rmsnorm_status_str(rn.OK) == "ok"
    for s in (rn.EINVAL, rn.EDTYPE, rn.EWORKSPACE, rn.EHIP, rn.ECONFIG, rn.ESCRATCH):
        assert rn.rmsnorm_status_str(s) not in ("ok", "unknown status")
    assert rn.rmsnorm_status_str(12345) == "unknown status"


FAKE = 1 << 20  # never dereferenced: every call below fails its checks first


@pytest.mark.parametrize("args,status", [
    (dict(dtype=7), rn.EDTYPE),
    (dict(M=-1), rn.EINVAL),
    (dict(N=0), rn.EINVAL),
    (dict(eps=-1.0), rn.EINVAL),
    (dict(eps=float("nan")), rn.EINVAL),
    (dict(eps=float("inf")), rn.EINVAL),
    (dict(x=None), rn.EINVAL),
    (dict(w=None), rn.EINVAL),
    (dict(y=None), rn.EINVAL),
    (dict(M=1 << 40, N=1 << 30), rn.EINVAL),
])
def test_fwd_argument_errors(args, status):
    a = dict(x=FAKE, w=FAKE, eps=1e-5, M=4, N=8, dtype=rn.F32, y=FAKE, rstd=None)
    a.update(args)
    rc = rn.lib.rmsnorm_fwd(a["x"], a["w"], a["eps"], a["M"], a["N"], a["dtype"], a["y"], a["rstd"], None)
    assert rc == status


def test_residual_argument_errors():
    # missing residual / dh with rows present; bad format; M = 0 is a no-op
    assert rn.lib.rmsnorm_fwd_residual(FAKE, None, FAKE, 1e-5, 4, 8, rn.BF16, FAKE, FAKE, None, None, None) == rn.EINVAL
    assert rn.lib.rmsnorm_fwd_residual(FAKE, FAKE, FAKE, 1e-5, 4, 8, rn.BF16, None, FAKE, None, None, None) == rn.EINVAL
    assert rn.lib.rmsnorm_fwd_residual(FAKE, FAKE, FAKE, 1e-5, 4, 8, 11, FAKE, FAKE, None, None, None) == rn.EDTYPE
    assert rn.lib.rmsnorm_fwd_residual(None, None, None, 1e-5, 0, 8, rn.F16, None, None, None, None, None) == rn.OK
    assert rn.lib.rmsnorm_bwd_residual(FAKE, FAKE, FAKE, None, FAKE, 4, 8, rn.F16, FAKE, FAKE, FAKE, 1 << 20,
                                       None, None) == rn.EINVAL
    assert rn.lib.rmsnorm_bwd_residual(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, rn.F16, FAKE, FAKE, None, 1 << 20,
                                       None, None) == rn.EWORKSPACE


def test_noalloc_argument_errors():
    # rmsnorm_bwd_noalloc checks its arguments before any HIP call (and before
    # looking up the static workspace)
    L = rn.lib
    assert L.rmsnorm_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, 4, 8, 9, FAKE, FAKE, None) == rn.EDTYPE
    assert L.rmsnorm_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, -1, 8, rn.BF16, FAKE, FAKE, None) == rn.EINVAL
    assert L.rmsnorm_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, 4, 0, rn.BF16, FAKE, FAKE, None) == rn.EINVAL
    assert L.rmsnorm_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, 4, 8, rn.BF16, FAKE, None, None) == rn.EINVAL
    for k in range(4):  # x, w, dy, rstd missing
        a = [FAKE] * 4
        a[k] = None
        assert L.rmsnorm_bwd_noalloc(*a, 4, 8, rn.BF16, FAKE, FAKE, None) == rn.EINVAL
    assert L.rmsnorm_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, 4, 8, rn.BF16, None, FAKE, None) == rn.EINVAL
    assert L.rmsnorm_bwd_noalloc(FAKE + 1, FAKE, FAKE, FAKE, 4, 8, rn.BF16, FAKE, FAKE, None) == rn.EINVAL
    assert L.rmsnorm_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, 4, 8, rn.BF16, FAKE, FAKE + 2, None) == rn.EINVAL
    assert rn.rmsnorm_status_str(rn.ESCRATCH) not in ("ok", "unknown status")


def test_unfused_baseline_argument_errors():
    # the unfused reference calls (the measurement library) take the 16-byte
    # vector layout only; all of these are rejected before any HIP call
    L = rn.bench_lib()
    assert L.rmsn_unfused_fwd(FAKE, FAKE, 1e-5, 4, 12, rn.BF16, FAKE, FAKE, None) == rn.EINVAL   # 24 B rows
    assert L.rmsn_unfused_fwd(FAKE + 2, FAKE, 1e-5, 4, 16, rn.BF16, FAKE, FAKE, None) == rn.EINVAL
    assert L.rmsn_unfused_fwd(FAKE, FAKE, 1e-5, 4, 16, rn.BF16, FAKE, None, None) == rn.EINVAL    # rstd required
    assert L.rmsn_unfused_fwd(FAKE, FAKE, -1.0, 4, 16, rn.BF16, FAKE, FAKE, None) == rn.EINVAL
    assert L.rmsn_unfused_fwd(FAKE, FAKE, 1e-5, 4, 16, 7, FAKE, FAKE, None) == rn.EDTYPE
    assert L.rmsn_unfused_fwd(None, None, 1e-5, 0, 16, rn.F32, None, None, None) == rn.OK
    assert L.rmsn_unfused_bwd_workspace_bytes(0, 64, rn.F32) == 0
    assert L.rmsn_unfused_bwd_workspace_bytes(4, 6, rn.F32) == rn.EINVAL
    need = L.rmsn_unfused_bwd_workspace_bytes(1000, 4096, rn.BF16)
    assert need == 256 * 4096 * 4 + 4096  # 256 row chunks of partial dW, then S (1000 floats, padded)
    assert L.rmsn_unfused_bwd(FAKE, FAKE, FAKE, FAKE, 1000, 4096, rn.BF16, FAKE, FAKE, FAKE, need - 1,
                              None) == rn.EWORKSPACE
    assert L.rmsn_unfused_bwd(FAKE, FAKE, FAKE, FAKE, 1000, 4096, rn.BF16, FAKE, FAKE, FAKE + 16, need,
                              None) == rn.EWORKSPACE
    assert L.rmsn_unfused_bwd(FAKE, FAKE, FAKE, None, 1000, 4096, rn.BF16, FAKE, FAKE, FAKE, need,
                              None) == rn.EINVAL
    assert L.rmsn_add(FAKE, FAKE, FAKE, 12, rn.BF16, None) == rn.EINVAL
    assert L.rmsn_add(FAKE, FAKE, FAKE, 16, 9, None) == rn.EDTYPE
    assert L.rmsn_add(None, None, None, 0, rn.F16, None) == rn.OK


def test_dtype_codes():
    import torch
    assert rn.dtype_code(torch.float32) == rn.F32 and rn.dtype_code(torch.bfloat16) == rn.BF16
    assert rn.dtype_code(torch.float16) == rn.F16
    assert rn.dtype_code(torch.bfloat16, torch.float32) == rn.BF16_WF32
    assert rn.dtype_code(torch.float16, torch.float32) == rn.F16_WF32
    with pytest.raises(ValueError):
        rn.dtype_code(torch.float32, torch.bfloat16)


@pytest.mark.parametrize("dtype", [rn.F16, rn.BF16_WF32, rn.F16_WF32])
def test_ladder_covers_new_formats(dtype):
    # 16-bit activations: the same shapes as bf16, except that the wide-row
    # backward prefetches only when the weights are 16-bit too, and that the
    # forward with fp32 weights runs a resident grid of two workgroups per CU
    # beyond 8 row blocks per CU (so that the weights stay in registers)
    for N, is_bwd in ((4096, 0), (4096, 1), (128, 0), (32768, 1), (32768, 0)):
        a = cfg(16384, N, dtype, is_bwd)
        b = cfg(16384, N, rn.BF16, is_bwd)
        if a["vector_path"] == 2 and dtype != rn.F16:
            assert a["prefetch"] == 0 and b["prefetch"] == 1
            a["prefetch"] = b["prefetch"]
            # 16384 rows of 32768 (a walk of 64): bf16 takes two workgroups per CU, fp32 weights keep one
            assert (a["grid"], b["grid"]) == (256, 512)
            a["grid"], a["partial_rows"] = b["grid"], b["partial_rows"]
        if not is_bwd and dtype != rn.F16 and N != 128:   # 128 columns: 1024 row blocks, 4 per CU
            assert a["grid"] == a["partial_rows"] == 512 and a["prefetch"] == 0 and b["grid"] > 512
            a["grid"], a["partial_rows"] = b["grid"], b["partial_rows"]
        assert a == b
    # fp32 weights: at most the resident workgroups; mid-size inputs keep the mid-size grid;
    # rows of under 128 lanes keep one block per workgroup
    if dtype != rn.F16:
        assert cfg(65536, 2048, dtype, 0)["grid"] == 65536 // cfg(65536, 2048, dtype, 0)["rows_per_wg"]
        assert cfg(1 << 20, 128, dtype, 0)["grid"] == cfg(1 << 20, 128, rn.BF16, 0)["grid"]
        assert cfg(16384, 4096, dtype, 0, blocks=1)["grid"] == 256
        c, d = cfg(2048, 4096, dtype, 0), cfg(2048, 4096, rn.BF16, 0)
        assert (c["grid"], c["prefetch"]) == (d["grid"], d["prefetch"]) == (768, 1)


def test_ladder_backward_grid_and_prefetch():
    """Partial rows (written and read once, 8 N bytes each) stay within 1/6 of
    the algorithmic bytes, never below one workgroup per CU. Rows of 512 or
    1024 lanes with 3/4 of them busy prefetch two row blocks with one
    workgroup per CU; other 1024-lane rows prefetch one block only when each
    workgroup walks at most 16 rows."""
    # bf16 4096 x 2048 (256 lanes): cap = 6*4096*2048 / 6 / (8*2048) = 512 -> 2 per CU
    assert cfg(4096, 2048, rn.BF16, 1)["grid"] == 512
    # bf16 1024 x 2048: cap 128 -> one per CU
    assert cfg(1024, 2048, rn.BF16, 1)["grid"] == 256
    # below one row block per CU: the row blocks
    assert cfg(100, 4096, rn.BF16, 1)["grid"] == 100
    # deep prefetch (register ring, walks outside the LDS path's 8 to 64 rows):
    # 512 lanes (4096 columns), 1024 lanes (8192, 7168 columns), fp32 4096
    for M, N, dt, lpr in ((1024, 4096, rn.BF16, 512), (65536, 4096, rn.BF16, 512), (65536, 8192, rn.BF16, 1024),
                          (1024, 7168, rn.BF16, 1024), (65536, 4096, rn.F32, 1024)):
        c = cfg(M, N, dt, 1)
        assert (c["lanes_per_row"], c["vecs_per_lane"], c["prefetch"], c["grid"], c["copy_mode"]) == \
            (lpr, 1, 2, 256, 0), (M, N)
    # 5120 columns: 640 whole-wavefront lanes over short walks (1536 rows), else
    # 1024 lanes (5/8 busy) under the short-walk rule (65536 rows: no prefetch)
    a, b = cfg(1536, 5120, rn.BF16, 1), cfg(65536, 5120, rn.BF16, 1)
    assert (a["lanes_per_row"], a["wg_threads"], a["grid"], a["prefetch"]) == (640, 640, 256, 2)
    assert (b["lanes_per_row"], b["grid"], b["prefetch"]) == (1024, 512, 0)
    # fp32 weights keep the power-of-two row: 1536 rows over 256 (the partial
    # cap) prefetch one block
    c = cfg(1536, 5120, rn.BF16_WF32, 1)
    assert (c["lanes_per_row"], c["grid"], c["prefetch"]) == (1024, 256, 1)
    # fp32, two vectors per lane: the short-walk rule; 3 or more never prefetch
    assert cfg(4096, 8192, rn.F32, 1)["prefetch"] == 1
    assert cfg(4096, 12288, rn.F32, 1)["prefetch"] == 0
    # rows of 64..256 lanes: 1024-lane workgroups, prefetching one block; 16-bit rows of
    # 64 or 128 lanes stop prefetching from walks of 4 row blocks (16384 x 1024: 4)
    for N, lpr, pf in ((512, 64, 1), (1024, 128, 0), (2048, 256, 1)):
        c = cfg(16384, N, rn.BF16, 1)
        assert (c["lanes_per_row"], c["wg_threads"], c["rows_per_wg"], c["prefetch"]) == (lpr, 1024, 1024 // lpr, pf)
    assert cfg(8192, 1024, rn.BF16, 1)["prefetch"] == 1           # a walk of 2 blocks
    assert cfg(65536, 512, rn.BF16, 1)["prefetch"] == 0           # 8 blocks
    assert cfg(65536, 512, rn.F32, 1)["prefetch"] == 1            # fp32 keeps it
    c = cfg(16384, 4096, rn.BF16, 1)
    assert (c["lanes_per_row"], c["wg_threads"], c["prefetch"], c["grid"]) == (512, 512, 2, 256)


@pytest.mark.parametrize("N,dtype,vpt,pf", [
    (16384, rn.BF16, 2, 1), (24576, rn.BF16, 3, 1), (32768, rn.BF16, 4, 1), (32768, rn.BF16_WF32, 4, 0),
    (32768, rn.F16, 4, 1), (20480, rn.F32, 5, 0), (32768, rn.F32, 8, 0),
])
def test_ladder_wide_rows(N, dtype, vpt, pf):
    """Backward rows of more than 1024 vectors: the wide-row kernel (1024 lanes,
    dW sums in LDS), one workgroup per compute unit."""
    c = cfg(4096, N, dtype, 1)
    assert (c["vector_path"], c["lanes_per_row"], c["vecs_per_lane"], c["wg_threads"], c["prefetch"]) == \
        (2, 1024, vpt, 1024, pf)
    assert c["grid"] == 256
    # fp32 up to 4 vectors per lane keeps the register kernel
    r = cfg(4096, 16384, rn.F32, 1)
    assert (r["vector_path"], r["vecs_per_lane"]) == (1, 4)
    # beyond what the LDS sums hold: the split-row kernel
    assert cfg(4096, 65536, rn.BF16, 1)["vector_path"] == 4
    assert cfg(4096, 36864, rn.F32, 1)["vector_path"] == 4


@pytest.mark.parametrize("M,N,dtype,blocks,K,vpt,grid", [
    (4096, 32768 + 8, rn.BF16, 2, 3, 2, 510),      # 4097 vectors: three slices of 1366, two members per CU
    (4096, 65536, rn.BF16, 2, 4, 2, 512),
    (4096, 65536, rn.BF16_WF32, 2, 4, 2, 512),
    (4096, 131072, rn.F16, 2, 8, 2, 512),
    (4096, 98304, rn.BF16, 2, 6, 2, 510),          # 85 groups of 6
    (4096, 262144, rn.BF16, 2, 16, 2, 512),        # 16 members of 2 vectors per lane
    (4096, 262144 + 8, rn.BF16, 1, 9, 4, 252),     # more than 16: one member per CU, 4 per lane
    (4096, 524288, rn.BF16, 1, 16, 4, 256),        # the widest split row
    (4096, 36864, rn.F32, 1, 2, 5, 256),           # fp32: the fewest members of one per CU
    (4096, 65536, rn.F32, 1, 2, 8, 256),
    (4096, 262144, rn.F32, 1, 8, 8, 256),
    (100, 65536, rn.BF16, 2, 4, 2, 400),           # a group per row
    (1, 65536, rn.BF16, 2, 4, 2, 4),
])
def test_ladder_split_rows(M, N, dtype, blocks, K, vpt, grid):
    """Backward rows wider than the wide-row kernel's LDS sums hold: K
    workgroups of 1024 lanes per row: 16-bit rows the fewest whose slices
    hold 2 vectors per lane while that is at most 16 members, else (and fp32
    rows) the fewest of up to 4 or 8; groups of K as many as stay resident (`blocks` per CU)
    and at most one per row; one partial dW row per group; no prefetch."""
    c = cfg(M, N, dtype, 1, blocks=blocks)
    assert (c["vector_path"], c["lanes_per_row"], c["vecs_per_lane"], c["wg_threads"], c["prefetch"]) == \
        (4, K * 1024, vpt, 1024, 0)
    assert c["rows_per_wg"] == 1 and c["copy_mode"] == 0
    assert (c["grid"], c["partial_rows"]) == (grid, grid // K)
    nvec = N * (4 if dtype == rn.F32 else 2) // 16
    slice_ = -(-nvec // K)
    assert (vpt - 1) * 1024 < slice_ <= vpt * 1024
    # the forward holds the same rows on one workgroup up to 16 vectors per lane
    if nvec <= 16384:
        f = cfg(M, N, dtype, 0)
        assert (f["vector_path"], f["lanes_per_row"], f["vecs_per_lane"], f["wg_threads"]) == \
            (1, 1024, -(-nvec // 1024), 1024)


def test_explicit_config_errors():
    """Explicit configurations are checked against the shape before any HIP call."""
    L, C = rn.lib, rn.rmsnorm_config

    def fwd(**kw):
        c = C(vector_path=1, lanes_per_row=128, vecs_per_lane=4, wg_threads=256, grid=8)
        for k, v in kw.items():
            setattr(c, k, v)
        return L.rmsnorm_fwd_with_config(FAKE, FAKE, 1e-5, 64, 4096, rn.BF16, FAKE, FAKE, c, None)

    assert fwd(stream_loads=2) == rn.ECONFIG
    assert fwd(grid=0) == rn.ECONFIG
    assert fwd(lanes_per_row=64) == rn.ECONFIG           # 64 x 4 vectors do not cover 512
    assert fwd(wg_threads=320) == rn.ECONFIG             # not whole rows
    assert fwd(vecs_per_lane=9, lanes_per_row=64) == rn.ECONFIG  # not built
    assert fwd(vector_path=2, lanes_per_row=1024, vecs_per_lane=1, wg_threads=1024) == rn.ECONFIG  # backward only
    assert fwd(vector_path=3) == rn.ECONFIG
    assert fwd(prefetch=2) == rn.ECONFIG
    assert fwd(kept_vecs=16) == rn.ECONFIG   # a field of the two-pass kernel only


@pytest.mark.parametrize("N,dtype", [(131072 + 8, rn.BF16), (65536 + 4, rn.F32), (1 << 20, rn.BF16_WF32),
                                     (1 << 22, rn.F16), (163840, rn.BF16), (163840 + 8, rn.BF16),
                                     (229376, rn.F16), (229376 + 8, rn.BF16), (81920, rn.F32), (81920 + 4, rn.F32),
                                     (163840, rn.F16_WF32), (163840 + 8, rn.BF16_WF32)])
def test_ladder_forward_two_pass_rows(N, dtype):
    """Forward rows wider than 16 vectors on each of 1024 lanes: the two-pass
    kernel (vector_path 5), one row per 1024-lane workgroup, a workgroup per
    row. Up to 20 vectors per lane: 16-bit rows in chunks of 4 with 16 kept
    in registers between the passes, fp32 activations or weights in chunks of
    2 with 14 kept (the most each keeps without spilling). Wider: 8 more held
    in LDS (copy_mode 1), 16-bit rows of 21-28 vectors per lane keeping 12,
    wider ones 16 in chunks of 2; fp32 14; fp32 weights 10."""
    v = -(-(N * (4 if dtype == rn.F32 else 2) // 16) // 1024)
    if dtype == rn.F32:
        want = (2, 14, 0) if v <= 20 else (2, 14, 1)
    elif dtype in (rn.BF16_WF32, rn.F16_WF32):
        want = (2, 14, 0) if v <= 20 else (2, 10, 1)
    else:
        want = (4, 16, 0) if v <= 20 else (4, 12, 1) if v <= 28 else (2, 16, 1)
    for M in (1, 300, 4096):
        c = cfg(M, N, dtype, 0)
        assert (c["vector_path"], c["lanes_per_row"], c["wg_threads"], c["prefetch"]) == (5, 1024, 1024, 0)
        assert (c["vecs_per_lane"], c["kept_vecs"], c["copy_mode"]) == want
        assert c["grid"] == M and c["rows_per_wg"] == 1
    # one vector per lane fewer: the register-held row
    r = cfg(64, 131072 if dtype != rn.F32 else 65536, dtype, 0)
    assert (r["vector_path"], r["vecs_per_lane"]) == (1, 16)


def test_ladder_forward_rows_beyond_32_bit_offsets():
    """The two-pass kernel addresses a row with 32-bit byte offsets: the one
    row size that does not fit (fp32, 2^30 columns = 4 GiB) takes the scalar
    kernel; one vector less still takes the two-pass kernel."""
    assert cfg(1, 1 << 30, rn.F32, 0)["vector_path"] == 0
    assert cfg(1, (1 << 30) - 4, rn.F32, 0)["vector_path"] == 5
    assert cfg(1, 1 << 30, rn.BF16, 0)["vector_path"] == 5


def test_explicit_loop_config_errors():
    """Two-pass configurations (vector_path 5) are forward only, on 1024 lanes,
    without prefetch, with copy_mode 0 or 1 (LDS-held vectors), and only for
    built (chunk, kept, LDS) shapes."""
    L, C = rn.lib, rn.rmsnorm_config
    M, N = 64, 262144

    def fwd(**kw):
        c = C(vector_path=5, lanes_per_row=1024, vecs_per_lane=8, wg_threads=1024, grid=64)
        for k, v in kw.items():
            setattr(c, k, v)
        return L.rmsnorm_fwd_with_config(FAKE, FAKE, 1e-5, M, N, rn.BF16, FAKE, FAKE, c, None)

    assert fwd(lanes_per_row=512) == rn.ECONFIG
    assert fwd(wg_threads=512) == rn.ECONFIG
    assert fwd(prefetch=1) == rn.ECONFIG
    assert fwd(vecs_per_lane=5) == rn.ECONFIG      # not built
    assert fwd(grid=0) == rn.ECONFIG
    assert fwd(kept_vecs=8) == rn.ECONFIG          # not built for chunks of 8
    assert fwd(copy_mode=1) == rn.ECONFIG          # nothing kept: no LDS-held shape built
    assert fwd(copy_mode=2) == rn.ECONFIG
    assert fwd(vecs_per_lane=2, kept_vecs=14, copy_mode=1) == rn.ECONFIG   # built for fp32 only
    assert fwd(vecs_per_lane=4, kept_vecs=14) == rn.ECONFIG   # not whole chunks
    assert fwd(vecs_per_lane=4, kept_vecs=-4) == rn.ECONFIG
    c = C(vector_path=5, lanes_per_row=1024, vecs_per_lane=8, wg_threads=1024, grid=4)
    assert L.rmsnorm_bwd_with_config(FAKE, FAKE, FAKE, FAKE, M, N, rn.BF16, FAKE, FAKE, FAKE, 1 << 30, c,
                                     None) == rn.ECONFIG


def test_explicit_split_config_errors():
    """Split-row configurations (vector_path 4) that cannot fit are refused
    before any HIP call: not whole groups, K outside 2..16, lanes not whole
    1024-lane members, slices wider than the kernel, no such kernel, the
    forward."""
    L, C = rn.lib, rn.rmsnorm_config
    M, N = 64, 65536

    def bwd(**kw):
        c = C(vector_path=4, lanes_per_row=2048, vecs_per_lane=4, wg_threads=1024, prefetch=1, grid=4)
        for k, v in kw.items():
            setattr(c, k, v)
        return L.rmsnorm_bwd_with_config(FAKE, FAKE, FAKE, FAKE, M, N, rn.BF16, FAKE, FAKE, FAKE, 1 << 30, c, None)

    assert bwd(grid=3) == rn.ECONFIG
    assert bwd(lanes_per_row=1024) == rn.ECONFIG
    assert bwd(lanes_per_row=17 * 1024, grid=17) == rn.ECONFIG
    assert bwd(lanes_per_row=1536) == rn.ECONFIG
    assert bwd(vecs_per_lane=3) == rn.ECONFIG      # 2048 x 3 vectors do not cover 8192
    assert bwd(vecs_per_lane=5) == rn.ECONFIG      # not built for 16-bit rows
    assert bwd(prefetch=2) == rn.ECONFIG
    assert bwd(copy_mode=1) == rn.ECONFIG
    assert bwd(wg_threads=512) == rn.ECONFIG
    assert bwd(stream_loads=1) == rn.ECONFIG
    c = C(vector_path=4, lanes_per_row=2048, vecs_per_lane=4, wg_threads=1024, prefetch=1, grid=4)
    assert L.rmsnorm_fwd_with_config(FAKE, FAKE, 1e-5, M, N, rn.BF16, FAKE, FAKE, c, None) == rn.ECONFIG


def test_fwd_empty_is_noop():
    assert rn.lib.rmsnorm_fwd(None, None, 1e-5, 0, 8, rn.F32, None, None, None) == rn.OK


@pytest.mark.parametrize("args,status", [
    (dict(dtype=9), rn.EDTYPE),
    (dict(M=-5), rn.EINVAL),
    (dict(dy=None), rn.EINVAL),
    (dict(rstd=None), rn.EINVAL),
    (dict(dx=None), rn.EINVAL),
    (dict(dw=None), rn.EINVAL),
    (dict(ws=None), rn.EWORKSPACE),
    (dict(ws=FAKE + 16), rn.EWORKSPACE),
])
def test_bwd_argument_errors(args, status):
    a = dict(x=FAKE, w=FAKE, dy=FAKE, rstd=FAKE, M=4, N=8, dtype=rn.BF16, dx=FAKE, dw=FAKE, ws=FAKE)
    a.update(args)
    rc = rn.lib.rmsnorm_bwd(a["x"], a["w"], a["dy"], a["rstd"], a["M"], a["N"], a["dtype"], a["dx"], a["dw"],
                            a["ws"], 1 << 20, None)
    assert rc == status


def test_workspace_query_argument_errors():
    assert rn.lib.rmsnorm_bwd_workspace_bytes(4, 8, 9) == rn.EDTYPE
    assert rn.lib.rmsnorm_bwd_workspace_bytes(-1, 8, rn.F32) == rn.EINVAL
    assert rn.lib.rmsnorm_bwd_workspace_bytes(0, 8, rn.F32) == 0


def cfg(M, N, dtype, is_bwd, aligned=1, cus=256, blocks=2):
    return rn.rmsnorm_select_config(M, N, dtype, is_bwd, aligned, cus, blocks).as_dict()


@pytest.mark.parametrize("N,dtype,is_bwd,lpr,vpt", [
    (128, rn.BF16, 0, 16, 1),      # QK-norm: 16 vectors -> 16 lanes, 4 rows per wavefront
    (128, rn.BF16, 1, 16, 1),
    (1024, rn.F32, 0, 64, 4),
    (1024, rn.F32, 1, 256, 1),
    (4096, rn.BF16, 0, 128, 4),
    (4096, rn.BF16, 1, 512, 1),
    (5120, rn.BF16, 0, 128, 5),    # 640 vectors: exactly 5 per lane on 128 lanes
    (10240, rn.BF16, 0, 256, 5),
    (2560, rn.F32, 0, 128, 5),
    (2560, rn.BF16, 0, 128, 3),    # 320 vectors: 64 lanes x 5 measured a tie; kept
    (5120, rn.BF16, 1, 640, 1),    # whole wavefronts (4096 rows: a short walk)
    (7168, rn.BF16, 0, 256, 4),
    (7168, rn.BF16, 1, 896, 1),    # 896 vectors, 4096 rows: the LDS-staged row on whole wavefronts
    (8192, rn.BF16, 0, 256, 4),
    (8192, rn.BF16, 1, 1024, 1),
    (32768, rn.BF16, 0, 1024, 4),
    (65536, rn.BF16, 0, 1024, 8),
    (16384, rn.F32, 1, 1024, 4),
    (8, rn.BF16, 0, 1, 1),
    (24, rn.BF16, 0, 4, 1),        # 3 vectors -> 4 lanes, one masked
])
def test_ladder_shapes(N, dtype, is_bwd, lpr, vpt):
    # the forward at 16384 rows, beyond the mid-size grids (which may change
    # the workgroup, not the row's shape)
    M = 4096 if is_bwd else 16384
    c = cfg(M, N, dtype, is_bwd)
    assert c["vector_path"] == 1
    assert (c["lanes_per_row"], c["vecs_per_lane"]) == (lpr, vpt)
    # backward rows of 64 to 256 lanes share 1024-lane workgroups
    assert c["wg_threads"] == (1024 if is_bwd and 64 <= lpr <= 256 else max(lpr, 256))
    # the LDS-staged backward for rows of 384 to 1024 vectors (4096 rows: a walk of 16)
    nv = N * (4 if dtype == rn.F32 else 2) // 16
    assert c["copy_mode"] == (1 if is_bwd and 384 <= nv <= 1024 else 0)
    # the forward streams rows of a wavefront or more with non-temporal loads
    # (every forward input here reaches the 4 MiB threshold but N = 8, 24)
    big = M * N * (4 if dtype == rn.F32 else 2) >= 4 << 20
    assert c["stream_loads"] == (1 if not is_bwd and lpr >= 64 and big else 0)
    # a decode step's few rows stay on plain loads
    assert cfg(16, N, dtype, 0)["stream_loads"] == 0
    assert c["rows_per_wg"] == c["wg_threads"] // lpr
    nvec = N * (4 if dtype == rn.F32 else 2) // 16
    assert (vpt - 1) * lpr < nvec <= vpt * lpr


@pytest.mark.parametrize("N,dtype,aligned,is_bwd", [(524288 + 8, rn.BF16, 1, 1), (524288 + 4, rn.F32, 1, 1),
                                                    (16385, rn.BF16, 1, 0), (20000, rn.F32, 0, 1),
                                                    (131072 + 8, rn.BF16, 0, 0)])
def test_ladder_scalar_cases(N, dtype, aligned, is_bwd):
    """The scalar kernel: rows the vector kernels cannot take that are wider
    than the element kernels hold (16384 columns), and backward rows wider
    than 16 split-row members of 4 16-bit or 8 fp32 vectors per lane hold."""
    c = cfg(100, N, dtype, is_bwd, aligned=aligned)
    assert c["vector_path"] == 0 and c["wg_threads"] == 256 and c["rows_per_wg"] == 1


ELEMENT_CASES = [
    # N, format, pointer alignment (1: 16 bytes), elements per access, forward (lanes, accesses), backward (...)
    (3, rn.BF16, 1, 1, (64, 1), (64, 1)), (13, rn.F32, 1, 1, (64, 1), (64, 1)), (255, rn.BF16, 1, 1, (64, 4), (64, 4)),
    (256, rn.BF16, 0, 1, (64, 4), (64, 4)), (257, rn.BF16, 1, 1, (64, 5), (64, 5)), (300, rn.BF16, 1, 4, (64, 2), (64, 2)),
    (1024, rn.BF16, 0, 1, (64, 16), (128, 8)), (1025, rn.F16, 1, 1, (128, 9), (128, 9)),
    (1500, rn.BF16, 1, 4, (128, 3), (128, 3)), (2050, rn.BF16, 1, 2, (256, 5), (256, 5)),
    (4095, rn.BF16, 1, 1, (256, 16), (512, 8)), (4096, rn.BF16, 0, 1, (256, 16), (512, 8)),
    (4100, rn.BF16, 1, 4, (512, 3), (512, 3)),        # 8200-byte rows: 8-byte accesses
    (4100, rn.BF16, 4, 2, (512, 5), (512, 5)),        # ... pointers only 4-byte aligned: 4-byte accesses
    (4100, rn.BF16_WF32, 1, 4, (512, 3), (512, 3)),   # fp32 weights: 16-byte weight accesses
    (4100, rn.F16_WF32, 2, 1, (512, 9), (512, 9)),
    (4098, rn.F32, 1, 2, (1024, 3), (512, 5)), (4104, rn.BF16, 8, 4, (512, 3), (512, 3)),
    (5001, rn.F32, 1, 1, (1024, 5), (512, 10)), (8192, rn.BF16, 8, 4, (512, 4), (1024, 2)),
    (10241, rn.BF16, 1, 1, (1024, 11), (1024, 11)), (16383, rn.F16, 1, 1, (1024, 16), (1024, 16)),
    (16384, rn.F16, 8, 4, (1024, 4), (1024, 4)), (16384, rn.F32, 8, 2, (1024, 8), (1024, 8)),
    (16384, rn.F32, 0, 1, (1024, 16), (1024, 16)),
]


@pytest.mark.parametrize("N,dtype,aligned,g,fwd,bwd", ELEMENT_CASES)
def test_ladder_element_cases(N, dtype, aligned, g, fwd, bwd):
    """Rows that are not a multiple of 16 bytes, or not 16-byte aligned, of up
    to 16384 columns: the element kernels. g elements per access (the largest
    power of two, up to 16 bytes of activations or weights, that divides N
    and the pointers' alignment); the fewest lanes, from 64, that keep a
    lane's share of the row within 16 elements and 32 bytes (forward) or 12
    elements and 40 bytes (backward), else 1024; ceil(N / (lanes g)) accesses
    per lane; no prefetch. The forward runs a workgroup per row; the backward
    is persistent on about 1024 lanes per CU (2 to 8 workgroups), within the
    partial-row and residency caps of the other row kernels."""
    es = 4 if dtype == rn.F32 else 2
    for is_bwd, (lanes, k) in ((0, fwd), (1, bwd)):
        c = cfg(16384, N, dtype, is_bwd, aligned=aligned, blocks=8)
        assert (c["vector_path"], c["lanes_per_row"], c["vecs_per_lane"], c["elems_per_access"], c["wg_threads"],
                c["rows_per_wg"], c["prefetch"], c["stream_loads"]) == (3, lanes, k, g, lanes, 1, 0, 0), c
        assert lanes * k * g >= N and k * g <= 16
        cap = max(256, 3 * 16384 * es // 48)
        assert c["grid"] == (min(max(2, min(8, 1024 // lanes)) * 256, cap, 8 * 256) if is_bwd else 16384)
        assert cfg(300, N, dtype, is_bwd, aligned=aligned)["grid"] == (256 if is_bwd else 300)
        assert cfg(16384, N, dtype, is_bwd, aligned=aligned, blocks=1)["grid"] == (256 if is_bwd else 16384)


def test_ladder_backward_single_workgroup_for_a_few_rows():
    """A few rows of the vector kernels: one workgroup walks them and writes dW
    itself (no combine) while M * N <= 16384 and the walk is at most 4 row
    blocks. The element kernels (not timed this way) keep their grid."""
    for M, N, dt in ((1, 4096, rn.BF16), (2, 4096, rn.BF16), (4, 4096, rn.BF16), (2, 8192, rn.BF16),
                     (8, 2048, rn.BF16), (4, 4096, rn.F32), (4, 2560, rn.BF16)):
        c = cfg(M, N, dt, 1)
        assert c["grid"] == c["partial_rows"] == 1, (M, N, c)
    for M, N, dt in ((5, 4096, rn.BF16), (3, 8192, rn.BF16), (12, 2048, rn.BF16), (300, 3, rn.BF16),
                     (17, 1024, rn.F32), (3, 5001, rn.BF16), (4, 257, rn.F32)):
        c = cfg(M, N, dt, 1)
        assert c["grid"] > 1, (M, N, c)


def test_ladder_grid_and_workspace_shape():
    # backward: two workgroups per compute unit, one fp32 partial row each
    c = cfg(16384, 2048, rn.BF16, 1, cus=256, blocks=2)
    assert c["grid"] == 512 and c["partial_rows"] == 512 and c["partial_stride"] == 2048 and c["prefetch"] == 1
    # ... capped by residency
    assert cfg(16384, 2048, rn.BF16, 1, cus=256, blocks=1)["grid"] == 256
    # ... fewer when the partial rows would exceed 1/6 of the bytes, never below the CUs
    assert cfg(2048, 4096, rn.BF16, 1, cus=256, blocks=2)["grid"] == 256
    # ... the wide-row kernel: one per compute unit
    assert cfg(4096, 32768, rn.BF16, 1, cus=256, blocks=2)["grid"] == 256
    # ... three per compute unit for rows narrower than a wavefront
    assert cfg(1 << 20, 128, rn.BF16, 1, cus=256, blocks=8)["grid"] == 768
    # ... two when three would leave some walks a block longer (1024 blocks: 6 -> 4 per CU)
    assert cfg(16384, 128, rn.BF16, 1, cus=256, blocks=8)["grid"] == 512
    assert cfg(131072, 128, rn.BF16, 1, cus=256, blocks=8)["grid"] == 768
    # ... 1024-lane workgroups that would each walk one row block: one per CU walking two
    assert cfg(4096, 1024, rn.BF16, 1, cus=256, blocks=8)["grid"] == 256
    assert cfg(6144, 1024, rn.BF16, 1, cus=256, blocks=8)["grid"] == 512
    # ... rows of 256 vectors over long walks: the LDS-staged kernel, one per CU
    c = cfg(65536, 2048, rn.BF16, 1, cus=256, blocks=8)
    assert (c["copy_mode"], c["lanes_per_row"], c["wg_threads"], c["grid"], c["prefetch"]) == (1, 256, 1024, 256, 2)
    assert cfg(16384, 2048, rn.BF16, 1, cus=256, blocks=8)["copy_mode"] == 0
    c = cfg(10, 4096, rn.BF16, 1, cus=256, blocks=2)      # fewer row blocks than workgroups wanted
    assert c["grid"] == (10 + c["rows_per_wg"] - 1) // c["rows_per_wg"]
    # forward: one row block per workgroup
    c = cfg(16384, 4096, rn.BF16, 0, cus=256, blocks=6)
    assert c["rows_per_wg"] == 2 and c["grid"] == 8192 and c["prefetch"] == 0
    assert cfg(1 << 24, 128, rn.BF16, 0)["grid"] == 1 << 20    # capped; workgroups then loop
    assert cfg(7, 13, rn.F32, 1)["partial_stride"] == 64
    # the ladder depends only on its arguments
    assert cfg(16384, 4096, rn.BF16, 1) == cfg(16384, 4096, rn.BF16, 1)


def test_select_config_argument_errors():
    with pytest.raises(rn.RmsnormError):
        rn.rmsnorm_select_config(4, 8, rn.F32, 0, 1, 0, 1)
    with pytest.raises(rn.RmsnormError):
        rn.rmsnorm_select_config(4, 8, 5, 0, 1, 256, 1)
    with pytest.raises(rn.RmsnormError):
        rn.rmsnorm_select_config(4, 8, rn.F32, 2, 1, 256, 1)


def test_binding_refuses_bad_tensors():
    """The binding passes tensors as raw pointers, so it checks them first: on
    the GPU, contiguous, of the format's dtype, large enough. These all fail
    before any call into the library (no GPU needed for the first ones)."""
    import torch
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    w = torch.zeros(8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="not on the GPU"):
        rn.rmsnorm_fwd(x, w, 1e-5, 4, 8, rn.BF16, x, None)
    with pytest.raises(TypeError, match="expected a torch tensor"):
        rn.rmsnorm_fwd([1, 2], FAKE, 1e-5, 4, 8, rn.BF16, FAKE, None)
    # integers (device addresses) and None pass through unchecked
    assert rn._arg(FAKE, "x", "act", rn.BF16, 32) == FAKE and rn._arg(None, "rstd", "f32", count=4) is None


def test_binding_tensor_checks_logic():
    """The checks themselves, on CPU tensors made to look like GPU ones."""
    import torch

    class FakeCuda(torch.Tensor):
        @property
        def is_cuda(self):
            return True

    def t(*shape, dtype=torch.bfloat16):
        return torch.zeros(*shape, dtype=dtype).as_subclass(FakeCuda)

    with pytest.raises(TypeError, match="dtype"):
        rn._arg(t(4, 8, dtype=torch.float32), "x", "act", rn.BF16, 32)
    with pytest.raises(TypeError, match="dtype"):
        rn._arg(t(8), "w", "weight", rn.BF16_WF32, 8)          # fp32 weights expected
    with pytest.raises(ValueError, match="elements"):
        rn._arg(t(3, 8), "y", "act", rn.BF16, 32)               # short output
    with pytest.raises(ValueError, match="not contiguous"):
        rn._arg(t(8, 4).t(), "x", "act", rn.BF16, 32)
    with pytest.raises(ValueError, match="bytes"):
        rn._arg(t(10, dtype=torch.float32), "workspace", nbytes=64)
    ok = t(4, 8)
    assert rn._arg(ok, "x", "act", rn.BF16, 32) == ok.data_ptr()
    assert rn._arg(ok, "x", "act", 9, 32) == ok.data_ptr()   # unknown format: the library reports it


@pytest.mark.parametrize("N,M,dtype,lanes,grid", [
    (2560, 16384, rn.BF16, 320, 512),     # 320 vectors: whole wavefronts, two per CU
    (3072, 65536, rn.F16, 384, 512),
    (3584, 65536, rn.BF16, 512, 256),     # 448: the 512-lane row (deep prefetch) is kept
    (4608, 1536, rn.BF16, 576, 256),      # 576-640: whole wavefronts on short walks only
    (4608, 65536, rn.BF16, 1024, 512),
    (6144, 65536, rn.BF16, 768, 256),     # 704-768: whole wavefronts, one per CU
    (5632, 65536, rn.F16, 704, 256),
    (7168, 65536, rn.BF16, 1024, 256),    # 832-960: the 1024-lane row is kept
    (2560, 65536, rn.F32, 1024, 512),     # fp32 keeps the power-of-two row
    (2560, 16384, rn.F16_WF32, 512, 512),
])
def test_ladder_whole_wavefront_rows(N, M, dtype, lanes, grid):
    """Backward rows of 257 to 1023 16-bit vectors run on whole wavefronts
    (a workgroup-sized row, depth-2 prefetch) where that measured faster than
    the next power of two; elsewhere the power-of-two row is kept. (Register
    ring; walks of 8 to 64 rows of 384 vectors or more take the LDS path.)"""
    c = cfg(M, N, dtype, 1)
    assert c["copy_mode"] == 0
    assert (c["vector_path"], c["lanes_per_row"], c["vecs_per_lane"], c["grid"]) == (1, lanes, 1, grid)
    if lanes & (lanes - 1):
        assert (c["wg_threads"], c["rows_per_wg"], c["prefetch"]) == (lanes, 1, 2)


@pytest.mark.parametrize("M,N,dtype,lanes", [
    (16384, 4096, rn.BF16, 512),          # the headline workload: a walk of 64
    (2048, 4096, rn.BF16, 512),           # a walk of 8
    (4096, 3072, rn.F16, 512),            # 384 vectors: 3/4 of 512 lanes
    (16384, 5120, rn.BF16, 640),          # whole wavefronts (16-bit activations)
    (8192, 6144, rn.F16, 768),
    (16384, 7168, rn.BF16, 896),
    (4096, 5120, rn.BF16_WF32, 640),
    (4096, 8192, rn.BF16, 1024),
    (4096, 2560, rn.F32, 1024),           # fp32: the power-of-two row
    (16384, 4096, rn.F32, 1024),
    (4096, 2048, rn.F32, 512),
])
def test_ladder_lds_path(M, N, dtype, lanes):
    """Backward rows of 384 to 1024 vectors over walks of 8 to 64 rows per
    workgroup take the LDS-staged kernel: two stages, one workgroup per CU."""
    c = cfg(M, N, dtype, 1)
    assert (c["copy_mode"], c["vector_path"], c["lanes_per_row"], c["vecs_per_lane"], c["wg_threads"],
            c["rows_per_wg"], c["prefetch"], c["grid"], c["partial_rows"]) == (1, 1, lanes, 1, lanes, 1, 2, 256, 256)


@pytest.mark.parametrize("M,N,dtype", [
    (1792, 4096, rn.BF16),                # a walk of 7
    (16385, 4096, rn.BF16),               # a walk of 65
    (16384, 2560, rn.BF16),               # 320 vectors
    (16384, 2048, rn.BF16),               # 256 vectors
    (4096, 16384, rn.BF16),               # 2048 vectors: the wide-row kernel
    (16384, 4100, rn.BF16),               # not a multiple of 16 bytes: the element kernels
])
def test_ladder_lds_path_boundaries(M, N, dtype):
    c = cfg(M, N, dtype, 1)
    assert c["copy_mode"] == 0
    assert cfg(M, N, dtype, 0)["copy_mode"] == 0   # never the forward
    assert cfg(16384, 4096, rn.BF16, 1, aligned=0)["copy_mode"] == 0   # unaligned pointers: element kernels


def test_explicit_whole_wavefront_config_checks():
    """Workgroup-sized rows through *_with_config are checked before any HIP
    call: the row must fit the lanes, hold one vector per lane, and the
    workgroup must be the row."""
    L, C = rn.lib, rn.rmsnorm_config

    def bwd(**kw):
        c = C(vector_path=1, lanes_per_row=640, vecs_per_lane=1, wg_threads=640, prefetch=2, grid=4)
        for k, v in kw.items():
            setattr(c, k, v)
        return L.rmsnorm_bwd_with_config(FAKE, FAKE, FAKE, FAKE, 8, 5120, rn.BF16, FAKE, FAKE, FAKE, 1 << 30, c, None)

    assert bwd(wg_threads=1280) == rn.ECONFIG               # two rows per workgroup: not built
    assert bwd(vecs_per_lane=2) == rn.ECONFIG               # one vector per lane only
    assert bwd(lanes_per_row=576, wg_threads=576) == rn.ECONFIG  # 576 lanes do not cover 640 vectors
    assert bwd(prefetch=0) == rn.ECONFIG                    # depths 1 and 2 are built


@pytest.mark.parametrize("dtype", [rn.F32, rn.BF16, rn.F16, rn.BF16_WF32, rn.F16_WF32])
def test_ladder_forward_mid_size_grid(dtype):
    """Forward inputs of 4 to 8 row blocks per compute unit on 256-lane
    workgroups: a grid of three per CU prefetching the next block; fewer row
    blocks keep one block per workgroup without prefetch, and so do more,
    except rows of 128 lanes or more with fp32 weights and 16-bit
    activations (two per CU). Where one 1024-lane workgroup per CU would walk
    exactly two blocks (fp32 2048 x 4096 and 4096 x 2048 here), that instead."""
    es = 4 if dtype == rn.F32 else 2
    w32 = dtype in (rn.BF16_WF32, rn.F16_WF32)
    for M, N in ((2048, 4096), (4096, 2048), (8192, 2048), (1024, 8192)):
        c = cfg(M, N, dtype, 0)
        rb = -(-M // c["rows_per_wg"])
        if c["wg_threads"] == 1024 and c["lanes_per_row"] < 1024:
            assert es == 4 and (c["grid"], c["prefetch"], rb) == (256, 1, 512), (M, N, c)
            continue
        mid = c["wg_threads"] <= 256 and 4 * 256 <= rb <= 8 * 256
        assert (c["grid"], c["prefetch"]) == ((768, 1) if mid else (rb, 0)), (M, N, c)
        if es == 2:
            assert mid
    for M, N in ((512, 4096), (16384, 4096), (16384, 2048)):
        c = cfg(M, N, dtype, 0)
        rb = -(-M // c["rows_per_wg"])
        wide = w32 and rb > 8 * 256 and c["lanes_per_row"] >= 128
        assert (c["grid"], c["prefetch"]) == ((512, 0) if wide else (rb, 0)), (M, N, c)
    # the residual-fused call keeps one block per workgroup (queried on the device, not here);
    # an explicit configuration keeps its own prefetch (checked with the other explicit tests)


def test_explicit_element_config_checks():
    """Element-kernel configurations through *_with_config are checked before
    any HIP call: 1024 lanes, 1 to 16 elements per lane covering the row, 1, 2,
    4 or 8 elements per access dividing N and the pointers' alignment, no
    prefetch, no streaming loads; elems_per_access is 0 on the other paths;
    a pointer not aligned to its element type is refused."""
    L, C = rn.lib, rn.rmsnorm_config

    def conf(kw):
        c = C(vector_path=3, lanes_per_row=1024, vecs_per_lane=8, elems_per_access=1, wg_threads=1024, grid=8)
        for k, v in kw.items():
            setattr(c, k, v)
        return c

    def fwd(**kw):
        return L.rmsnorm_fwd_with_config(FAKE, FAKE, 1e-5, 64, 4100, rn.BF16, FAKE, FAKE, conf(kw), None)

    def bwd(N, **kw):
        return L.rmsnorm_bwd_with_config(FAKE, FAKE, FAKE, FAKE, 64, N, rn.BF16, FAKE, FAKE, FAKE, 1 << 30,
                                         conf(kw), None)

    def bwd_res(N, **kw):
        return L.rmsnorm_bwd_residual(FAKE, FAKE, FAKE, FAKE, FAKE, 64, N, rn.BF16, FAKE, FAKE, FAKE, 1 << 30,
                                      conf(kw), None)

    assert fwd(vecs_per_lane=4) == rn.ECONFIG       # 4096 elements do not cover 4100
    assert fwd(vecs_per_lane=17) == rn.ECONFIG      # beyond 16
    assert fwd(vecs_per_lane=0) == rn.ECONFIG
    assert fwd(lanes_per_row=512) == rn.ECONFIG
    assert fwd(wg_threads=512) == rn.ECONFIG
    assert fwd(prefetch=1) == rn.ECONFIG
    assert fwd(prefetch=-1) == rn.ECONFIG
    assert fwd(stream_loads=1) == rn.ECONFIG
    assert fwd(vector_path=4) == rn.ECONFIG
    assert fwd(elems_per_access=3) == rn.ECONFIG
    assert fwd(elems_per_access=8, vecs_per_lane=1) == rn.ECONFIG     # 8 does not divide 4100
    assert fwd(elems_per_access=4, vecs_per_lane=8) == rn.ECONFIG     # 32 elements per lane
    assert fwd(elems_per_access=4, vecs_per_lane=1) == rn.ECONFIG     # 4096 elements do not cover 4100
    assert L.rmsnorm_fwd_with_config(FAKE, FAKE, 1e-5, 64, 4100, rn.BF16, FAKE + 4, FAKE,
                                     conf(dict(elems_per_access=4, vecs_per_lane=2)), None) == rn.ECONFIG
    assert L.rmsnorm_fwd_with_config(FAKE, FAKE + 8, 1e-5, 64, 4100, rn.BF16_WF32, FAKE, FAKE,
                                     conf(dict(elems_per_access=4, vecs_per_lane=2)), None) == rn.ECONFIG
    assert L.rmsnorm_fwd_with_config(FAKE, FAKE, 1e-5, 64, 4096, rn.BF16, FAKE, FAKE,
                                     C(vector_path=1, lanes_per_row=512, vecs_per_lane=1, elems_per_access=2,
                                       grid=8), None) == rn.ECONFIG
    # pointers not aligned to their element type
    assert L.rmsnorm_fwd(FAKE + 1, FAKE, 1e-5, 64, 4100, rn.BF16, FAKE, FAKE, None) == rn.EINVAL
    assert L.rmsnorm_fwd(FAKE, FAKE + 2, 1e-5, 64, 4100, rn.BF16_WF32, FAKE, FAKE, None) == rn.EINVAL
    assert L.rmsnorm_fwd(FAKE, FAKE, 1e-5, 64, 4100, rn.F32, FAKE + 2, FAKE, None) == rn.EINVAL
    assert L.rmsnorm_fwd(FAKE, FAKE, 1e-5, 64, 4096, rn.BF16, FAKE, FAKE + 2, None) == rn.EINVAL     # rstd
    assert L.rmsnorm_bwd(FAKE, FAKE, FAKE, FAKE + 2, 64, 4096, rn.BF16, FAKE, FAKE, FAKE, 1 << 30,
                         None) == rn.EINVAL                                                         # rstd
    assert L.rmsnorm_bwd(FAKE, FAKE, FAKE, FAKE, 64, 4096, rn.BF16, FAKE, FAKE + 2, FAKE, 1 << 30,
                         None) == rn.EINVAL                                                         # dW
    assert L.rmsnorm_bwd(FAKE, FAKE, FAKE, FAKE, 0, 4096, rn.BF16, FAKE, FAKE + 2, FAKE, 1 << 30,
                         None) == rn.EINVAL                                                         # dW, M = 0
    assert bwd(4100, vecs_per_lane=5, prefetch=1) == rn.ECONFIG
    assert bwd(14000, vecs_per_lane=13) == rn.ECONFIG                # 13312 elements do not cover 14000
    assert bwd_res(4100, vecs_per_lane=5, stream_loads=1) == rn.ECONFIG
    assert bwd_res(4100, vecs_per_lane=5, lanes_per_row=256) == rn.ECONFIG


def test_lds_copy_mode_configurations():
    """Explicit configurations with copy_mode 1 (the LDS-staged backward):
    built shapes get past every check to the launch (which fails here, with
    no GPU); unbuilt stage counts, depths outside 2..8, several vectors per
    lane, other paths and the forward are refused before any HIP call."""
    import ctypes

    def rc(dt, N, is_bwd=1, **kw):
        d = dict(vector_path=1, lanes_per_row=256, vecs_per_lane=1, wg_threads=1024, prefetch=2, copy_mode=1,
                 grid=3)
        d.update(kw)
        c = rn.rmsnorm_config(**d)
        if is_bwd:
            return rn.lib.rmsnorm_bwd_with_config(FAKE, FAKE, FAKE, FAKE, 63, N, dt, FAKE, FAKE, FAKE, 1 << 30,
                                                  ctypes.byref(c), None)
        return rn.lib.rmsnorm_fwd_with_config(FAKE, FAKE, 1e-6, 63, N, dt, FAKE, FAKE, ctypes.byref(c), None)

    for dt, N, kw in ((rn.F32, 524, {}), (rn.BF16, 2128, dict(lanes_per_row=512, wg_threads=512, prefetch=8)),
                      (rn.BF16_WF32, 5120, dict(lanes_per_row=640, wg_threads=640, prefetch=3)),
                      (rn.F16, 8192, dict(lanes_per_row=1024, wg_threads=1024, prefetch=4))):
        assert rc(dt, N, **kw) == rn.EHIP, (dt, N, kw)  # valid: reaches the launch
    bad = [dict(lanes_per_row=512, wg_threads=512, prefetch=5), dict(lanes_per_row=512, wg_threads=512, prefetch=1),
           dict(lanes_per_row=512, wg_threads=512, prefetch=9), dict(lanes_per_row=256, vecs_per_lane=2),
           dict(lanes_per_row=512, wg_threads=1024, prefetch=4), dict(copy_mode=2), dict(copy_mode=-1),
           dict(vector_path=2, lanes_per_row=1024, wg_threads=1024), dict(vector_path=0)]
    for kw in bad:
        assert rc(rn.BF16, 2128, **kw) == rn.ECONFIG, kw
    assert rc(rn.BF16, 4096, is_bwd=0, lanes_per_row=128, vecs_per_lane=4, wg_threads=256) == rn.ECONFIG


@pytest.mark.parametrize("M,N,dtype,vpt,pf,grid", [
    (16384, 16384, rn.BF16, 2, 0, 512),   # a walk of 64: two per CU, no prefetch
    (32768, 24576, rn.F16, 3, 0, 512),
    (16384, 32768, rn.BF16, 4, 1, 512),   # 4 vectors per lane keep the prefetch
    (8192, 16384, rn.BF16, 2, 1, 256),    # a walk of 32: one prefetching workgroup per CU
    (16384, 16384, rn.BF16_WF32, 2, 0, 256),  # fp32 weights: one per CU, no prefetch
    (16384, 32768, rn.F32, 8, 0, 256),
])
def test_ladder_wide_rows_long_walks(M, N, dtype, vpt, pf, grid):
    """Wide rows with 16-bit activations and weights over walks of 64 rows per
    CU or more: two workgroups per CU (beyond residency at 4 vectors per
    lane), prefetch off at 2-3 vectors per lane."""
    c = cfg(M, N, dtype, 1, blocks=1)
    assert (c["vector_path"], c["vecs_per_lane"], c["prefetch"], c["grid"]) == (2, vpt, pf, grid)


@pytest.mark.parametrize("M,N,dtype,walk", [
    (32768, 8192, rn.BF16, True), (65536, 8192, rn.F16, True), (131072, 8192, rn.BF16, True),
    (24576, 8192, rn.BF16, False),       # fewer rows: a row per 256-lane workgroup
    (32768, 4096, rn.F32, False),        # fp32 rows of 1024 vectors keep it
    (32768, 8192, rn.BF16_WF32, False),  # fp32 weights: the resident grid
    (32768, 16384, rn.BF16, False), (65536, 4096, rn.BF16, False),
])
def test_ladder_forward_row_walk(M, N, dtype, walk):
    """Plain forward rows of 1024 16-bit vectors over 32768 rows or more: one
    row per 1024-lane workgroup, each walking two rows with the next one's
    loads issued first; everything else keeps its shape."""
    c = cfg(M, N, dtype, 0)
    got = (c["lanes_per_row"], c["vecs_per_lane"], c["wg_threads"], c["prefetch"], c["grid"])
    if walk:
        assert got == (1024, 1, 1024, 1, M // 2)
    else:
        assert got[0] != 1024 or got[3] == 0


def test_ladder_forward_row_walk_grid_cap():
    """The walk's grid stays within 2^20 workgroups; beyond that each walks more rows."""
    c = cfg(4 << 20, 8192, rn.BF16, 0)
    assert (c["lanes_per_row"], c["prefetch"], c["grid"]) == (1024, 1, 1 << 20)


@pytest.mark.parametrize("M,N,dtype,wide", [
    (8192, 512, rn.BF16, True), (8192, 1024, rn.BF16, True), (4096, 4096, rn.BF16, True),
    (2048, 8192, rn.BF16, True), (8192, 256, rn.F32, True), (8192, 512, rn.F16, True),
    (8192, 512, rn.BF16_WF32, True), (7168, 512, rn.BF16, True),
    (6144, 512, rn.BF16, False),     # 6 blocks per CU: three 256-lane walkers per CU split evenly
    (4096, 512, rn.BF16, False),
    (8192, 2048, rn.BF16, False),    # 64-lane rows of 4 vectors keep the 256-lane grid
    (8192, 1024, rn.F16, False),     # no 1024-lane fp16 kernel of 2 vectors per lane
    (16384, 4096, rn.BF16, False),   # beyond the mid-size range
])
def test_ladder_forward_mid_wide(M, N, dtype, wide):
    """Mid-size plain forward inputs of more than 6 row blocks per CU: one
    prefetching 1024-lane workgroup per CU walking two blocks."""
    c = cfg(M, N, dtype, 0)
    if wide:
        assert (c["wg_threads"], c["rows_per_wg"], c["prefetch"], c["grid"]) == \
            (1024, 1024 // c["lanes_per_row"], 1, 256)
    else:
        assert c["wg_threads"] != 1024 or c["lanes_per_row"] == 1024


@pytest.mark.parametrize("M,N,dtype,wide", [
    (24576, 512, rn.BF16, True), (32768, 512, rn.F16, True), (131072, 512, rn.BF16, True),
    (32768, 256, rn.F32, True), (32768, 512, rn.BF16_WF32, True),
    (16384, 512, rn.F16, False),    # 16 blocks of 256 lanes per CU: a tie, not taken
    (32768, 384, rn.BF16, False),   # 48 vectors on 64 lanes
    (32768, 1024, rn.BF16, False),  # two vectors per lane
])
def test_ladder_forward_rows64(M, N, dtype, wide):
    """Plain forward rows of exactly 64 vectors beyond 16 row blocks of 256
    lanes per CU: 16 rows per 1024-lane workgroup, one block each."""
    c = cfg(M, N, dtype, 0)
    assert c["lanes_per_row"] == 64
    if wide:
        assert (c["wg_threads"], c["rows_per_wg"], c["prefetch"], c["grid"]) == (1024, 16, 0, M // 16)
    else:
        assert c["wg_threads"] == 256


@pytest.mark.parametrize("M,N,dtype,wide", [
    (10240, 512, rn.BF16, True), (16384, 512, rn.BF16, True), (20480, 512, rn.BF16, True),
    (16384, 1024, rn.BF16, True), (12288, 256, rn.F32, True), (16384, 512, rn.F32, True),
    (24576, 512, rn.BF16, False),   # beyond 20 blocks per CU: the 1024-lane grid
    (18432, 1024, rn.BF16, False),  # two vectors per lane: up to 16 blocks per CU
    (16384, 2048, rn.BF16, False),  # four vectors per lane
    (16384, 512, rn.F16, False),    # no 512-lane fp16 kernel
    (8192, 512, rn.BF16, False),    # the mid-size range (its 1024-lane grid)
])
def test_ladder_forward_rows64_512(M, N, dtype, wide):
    """64-lane forward rows of one vector from 9 to 20 row blocks of 256 lanes
    per CU (of two vectors: to 16): 512-lane workgroups, three per CU,
    prefetching."""
    c = cfg(M, N, dtype, 0)
    assert c["lanes_per_row"] == 64
    got = (c["wg_threads"], c["rows_per_wg"], c["prefetch"], c["grid"])
    if wide:
        assert got == (512, 8, 1, 768)
    else:
        assert got[0] != 512


@pytest.mark.parametrize("M,N,dtype,taken", [
    (40960, 128, rn.BF16, True), (65536, 128, rn.BF16, True), (98304, 128, rn.BF16, True),
    (131072, 64, rn.BF16, True), (65536, 64, rn.F32, True), (32768, 256, rn.BF16, True), (65536, 128, rn.F16, True),
    (32768, 128, rn.BF16, False),     # 8 blocks per CU
    (131072, 128, rn.BF16, False),    # 32 blocks per CU
    (1 << 20, 128, rn.BF16, False),   # QK-norm rows
    (65536, 128, rn.BF16_WF32, False),
])
def test_ladder_forward_narrow_grid(M, N, dtype, taken):
    """Forward rows narrower than a wavefront from 9 to 24 row blocks per CU:
    a prefetching grid of four workgroups per CU."""
    c = cfg(M, N, dtype, 0)
    assert c["lanes_per_row"] < 64 and c["wg_threads"] == 256
    rb = -(-M // c["rows_per_wg"])
    if taken:
        assert (c["grid"], c["prefetch"]) == (1024, 1)
    else:
        assert (c["grid"], c["prefetch"]) == (rb, 0)
