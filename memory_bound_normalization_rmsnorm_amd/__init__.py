"""Python binding of the gfx950 RMSNorm library (``librmsnorm_mi355x.so``).

Argument marshalling only: every function forwards to the C entry point of
the same name declared in ``include/rmsnorm.h``; the roofline probes
(``include/rmsnorm_probe.h``) and the unfused reference kernels
(``include/rmsnorm_baseline.h``) live in a separate measurement library,
``librmsnorm_mi355x_bench.so``, loaded on their first use, so the product
library carries no measurement code. Pointers may be given as integers (device
addresses) or as torch tensors (their ``data_ptr()``); ``stream`` may be an
integer hipStream_t, a ``torch.cuda.Stream``, or None for torch's current
stream. A non-zero status raises ``RmsnormError``.

torch is imported first so that the library binds to the HIP runtime torch
already loaded (one runtime per process). Importing this package fails when
the library has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library links against)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "librmsnorm_mi355x.so"
# RMSNORM_MI355X_LIB selects another build of the same library (for example
# one compiled with different flags, to compare variants); default: in-tree.
LIB_PATH = os.environ.get("RMSNORM_MI355X_LIB") or os.path.join(_HERE, LIB_NAME)
BENCH_LIB_NAME = "librmsnorm_mi355x_bench.so"
BENCH_LIB_PATH = os.path.join(_HERE, BENCH_LIB_NAME)

F32 = 0
BF16 = 1
F16 = 2
BF16_WF32 = 3
F16_WF32 = 4

OK = 0
EINVAL = -1
EDTYPE = -2
EWORKSPACE = -3
EHIP = -4
ECONFIG = -5
ESCRATCH = -6
NOALLOC_SCRATCH_BYTES = 32 << 20  # RMSN_NOALLOC_SCRATCH_BYTES


class RmsnormError(RuntimeError):
    def __init__(self, name: str, status: int, text: str):
        super().__init__(f"{name} failed: {text} (status {status})")
        self.status = status


class rmsnorm_config(ctypes.Structure):
    _fields_ = [
        ("vector_path", ctypes.c_int32),
        ("lanes_per_row", ctypes.c_int32),
        ("vecs_per_lane", ctypes.c_int32),
        ("wg_threads", ctypes.c_int32),
        ("rows_per_wg", ctypes.c_int32),
        ("prefetch", ctypes.c_int32),
        ("stream_loads", ctypes.c_int32),
        ("elems_per_access", ctypes.c_int32),
        ("copy_mode", ctypes.c_int32),
        ("kept_vecs", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("partial_rows", ctypes.c_int64),
        ("partial_stride", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc --offload-arch=gfx950). There is no CPU or eager fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    cfgp = ctypes.POINTER(rmsnorm_config)
    sig = {
        "rmsnorm_fwd": (i32, [vp, vp, f32, i64, i64, i32, vp, vp, vp]),
        "rmsnorm_fwd_with_config": (i32, [vp, vp, f32, i64, i64, i32, vp, vp, cfgp, vp]),
        "rmsnorm_bwd_workspace_bytes": (i64, [i64, i64, i32]),
        "rmsnorm_bwd": (i32, [vp, vp, vp, vp, i64, i64, i32, vp, vp, vp, sz, vp]),
        "rmsnorm_bwd_with_config": (i32, [vp, vp, vp, vp, i64, i64, i32, vp, vp, vp, sz, cfgp, vp]),
        "rmsnorm_bwd_rows": (i32, [vp, vp, vp, vp, i64, i64, i32, vp, vp, sz, ctypes.POINTER(i64), vp]),
        "rmsnorm_bwd_noalloc": (i32, [vp, vp, vp, vp, i64, i64, i32, vp, vp, vp]),
        "rmsnorm_fwd_residual": (i32, [vp, vp, vp, f32, i64, i64, i32, vp, vp, vp, cfgp, vp]),
        "rmsnorm_bwd_residual": (i32, [vp, vp, vp, vp, vp, i64, i64, i32, vp, vp, vp, sz, cfgp, vp]),
        "rmsnorm_bwd_combine": (i32, [vp, i64, i64, vp, vp]),
        "rmsnorm_status_str": (ctypes.c_char_p, [i32]),
        "rmsnorm_select_config": (i32, [i64, i64, i32, i32, i32, i32, i32, cfgp]),
        "rmsnorm_query_config": (i32, [i64, i64, i32, i32, cfgp]),
        "rmsnorm_build_info": (ctypes.c_char_p, []),
    }
    _bind(lib, sig)
    return lib


def _bind(lib, sig):
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


lib = _load()
_bench = None


def bench_lib() -> ctypes.CDLL:
    """The measurement library (roofline probes, unfused reference kernels),
    loaded on first use. Raises ImportError when it has not been built."""
    global _bench
    if _bench is None:
        if not os.path.exists(BENCH_LIB_PATH):
            raise ImportError(f"{BENCH_LIB_PATH} is not built; `python -c 'import __graft_entry__ as g; g.build()'` "
                              "builds it beside the product library.")
        b = ctypes.CDLL(BENCH_LIB_PATH)
        vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        _bind(b, {
            "rmsn_probe_copy": (i32, [vp, vp, sz, i64, i32, vp]),
            "rmsn_probe_write": (i32, [vp, sz, i64, i32, vp]),
            "rmsn_probe_read": (i32, [vp, sz, i64, i32, vp, vp]),
            "rmsn_probe_add": (i32, [vp, vp, vp, sz, i64, i32, vp]),
            "rmsn_unfused_fwd": (i32, [vp, vp, f32, i64, i64, i32, vp, vp, vp]),
            "rmsn_unfused_bwd_workspace_bytes": (i64, [i64, i64, i32]),
            "rmsn_unfused_bwd": (i32, [vp, vp, vp, vp, i64, i64, i32, vp, vp, vp, sz, vp]),
            "rmsn_add": (i32, [vp, vp, vp, i64, i32, vp]),
        })
        _bench = b
    return _bench


# entry points of the product library (include/rmsnorm.h)
EXPORTED = (
    "rmsnorm_fwd", "rmsnorm_fwd_with_config", "rmsnorm_bwd_workspace_bytes", "rmsnorm_bwd",
    "rmsnorm_bwd_with_config", "rmsnorm_bwd_rows", "rmsnorm_bwd_combine", "rmsnorm_fwd_residual",
    "rmsnorm_bwd_residual", "rmsnorm_bwd_noalloc", "rmsnorm_status_str",
    "rmsnorm_select_config", "rmsnorm_query_config", "rmsnorm_build_info",
)
# entry points of the measurement library (include/rmsnorm_probe.h, include/rmsnorm_baseline.h)
BENCH_EXPORTED = (
    "rmsn_probe_copy", "rmsn_probe_write", "rmsn_probe_read", "rmsn_probe_add",
    "rmsn_unfused_fwd", "rmsn_unfused_bwd_workspace_bytes", "rmsn_unfused_bwd", "rmsn_add",
)


def _ptr(p):
    if p is None:
        return None
    if isinstance(p, int):
        return p
    return p.data_ptr()


# activation and weight torch dtypes of each format code
_ACT = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16, BF16_WF32: torch.bfloat16,
        F16_WF32: torch.float16}
_WEIGHT = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16, BF16_WF32: torch.float32,
           F16_WF32: torch.float32}


def _arg(p, what: str, kind: str = "raw", code=None, count=None, nbytes=None):
    """Pointer of an argument. Integers (device addresses) and None pass
    through. A tensor must be a contiguous GPU tensor of the format's dtype
    (kind "act", "weight" or "f32") holding at least `count` elements (or
    `nbytes` bytes): the C entry points take raw pointers and cannot check
    what they point to, and a short buffer would be read or written out of
    bounds."""
    if p is None or isinstance(p, int):
        return p
    if not isinstance(p, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor, a device address or None, got {type(p).__name__}")
    if not p.is_cuda:
        raise ValueError(f"{what}: tensor is on {p.device}, not on the GPU")
    if not p.is_contiguous():
        raise ValueError(f"{what}: tensor is not contiguous (row-major [M][N] is required)")
    want = {"act": _ACT.get(code), "weight": _WEIGHT.get(code), "f32": torch.float32}.get(kind)
    if want is not None and p.dtype != want:
        raise TypeError(f"{what}: dtype {p.dtype}, format {code} needs {want}")
    if count is not None and count >= 0 and p.numel() < count:
        raise ValueError(f"{what}: {p.numel()} elements, the call needs {count}")
    if nbytes is not None and nbytes >= 0 and p.numel() * p.element_size() < nbytes:
        raise ValueError(f"{what}: {p.numel() * p.element_size()} bytes, the call needs {nbytes}")
    return p.data_ptr()


def _mn(M, N):
    return int(M) * int(N) if int(M) >= 0 and int(N) >= 0 else -1


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(name: str, rc: int) -> None:
    if rc != OK:
        raise RmsnormError(name, rc, rmsnorm_status_str(rc))


def dtype_code(torch_dtype, weight_dtype=None) -> int:
    """rmsn_dtype code of an activation torch dtype and (optionally) a weight dtype."""
    weight_dtype = weight_dtype or torch_dtype
    codes = {(torch.float32, torch.float32): F32, (torch.bfloat16, torch.bfloat16): BF16,
             (torch.float16, torch.float16): F16, (torch.bfloat16, torch.float32): BF16_WF32,
             (torch.float16, torch.float32): F16_WF32}
    try:
        return codes[(torch_dtype, weight_dtype)]
    except KeyError:
        raise ValueError(f"unsupported formats {torch_dtype} / {weight_dtype}") from None


def rmsnorm_status_str(status: int) -> str:
    return lib.rmsnorm_status_str(int(status)).decode()


def rmsnorm_build_info() -> str:
    return lib.rmsnorm_build_info().decode()


def rmsnorm_fwd(x, w, eps, M, N, dtype, y, rstd, stream=None) -> None:
    mn = _mn(M, N)
    _check("rmsnorm_fwd", lib.rmsnorm_fwd(_arg(x, "x", "act", dtype, mn), _arg(w, "w", "weight", dtype, int(N)),
                                          float(eps), int(M), int(N), int(dtype), _arg(y, "y", "act", dtype, mn),
                                          _arg(rstd, "rstd", "f32", count=int(M)), _stream(stream)))


def rmsnorm_fwd_with_config(x, w, eps, M, N, dtype, y, rstd, cfg: rmsnorm_config, stream=None) -> None:
    mn = _mn(M, N)
    _check("rmsnorm_fwd_with_config",
           lib.rmsnorm_fwd_with_config(_arg(x, "x", "act", dtype, mn), _arg(w, "w", "weight", dtype, int(N)),
                                       float(eps), int(M), int(N), int(dtype), _arg(y, "y", "act", dtype, mn),
                                       _arg(rstd, "rstd", "f32", count=int(M)), ctypes.byref(cfg), _stream(stream)))


def rmsnorm_bwd_workspace_bytes(M, N, dtype) -> int:
    n = lib.rmsnorm_bwd_workspace_bytes(int(M), int(N), int(dtype))
    _check("rmsnorm_bwd_workspace_bytes", n if n < 0 else OK)
    return int(n)


def rmsnorm_bwd(x, w, dy, rstd, M, N, dtype, dx, dw, workspace, workspace_bytes, stream=None) -> None:
    mn = _mn(M, N)
    _check("rmsnorm_bwd", lib.rmsnorm_bwd(_arg(x, "x", "act", dtype, mn), _arg(w, "w", "weight", dtype, int(N)),
                                          _arg(dy, "dy", "act", dtype, mn), _arg(rstd, "rstd", "f32", count=int(M)),
                                          int(M), int(N), int(dtype), _arg(dx, "dx", "act", dtype, mn),
                                          _arg(dw, "dw", "f32", count=int(N)),
                                          _arg(workspace, "workspace", nbytes=int(workspace_bytes)),
                                          int(workspace_bytes), _stream(stream)))


def rmsnorm_bwd_noalloc(x, w, dy, rstd, M, N, dtype, dx, dw, stream=None) -> None:
    """rmsnorm_bwd with its dW partial rows in the library's static device
    array instead of a caller's workspace (no allocation; RMSN_ESCRATCH when
    the shape needs more than NOALLOC_SCRATCH_BYTES)."""
    mn = _mn(M, N)
    _check("rmsnorm_bwd_noalloc",
           lib.rmsnorm_bwd_noalloc(_arg(x, "x", "act", dtype, mn), _arg(w, "w", "weight", dtype, int(N)),
                                   _arg(dy, "dy", "act", dtype, mn), _arg(rstd, "rstd", "f32", count=int(M)),
                                   int(M), int(N), int(dtype), _arg(dx, "dx", "act", dtype, mn),
                                   _arg(dw, "dw", "f32", count=int(N)), _stream(stream)))


def rmsnorm_bwd_with_config(x, w, dy, rstd, M, N, dtype, dx, dw, workspace, workspace_bytes,
                            cfg: rmsnorm_config, stream=None) -> None:
    mn = _mn(M, N)
    _check("rmsnorm_bwd_with_config",
           lib.rmsnorm_bwd_with_config(_arg(x, "x", "act", dtype, mn), _arg(w, "w", "weight", dtype, int(N)),
                                       _arg(dy, "dy", "act", dtype, mn), _arg(rstd, "rstd", "f32", count=int(M)),
                                       int(M), int(N), int(dtype), _arg(dx, "dx", "act", dtype, mn),
                                       _arg(dw, "dw", "f32", count=int(N)),
                                       _arg(workspace, "workspace", nbytes=int(workspace_bytes)),
                                       int(workspace_bytes), ctypes.byref(cfg), _stream(stream)))


def rmsnorm_fwd_residual(x, res, w, eps, M, N, dtype, h, y, rstd, cfg=None, stream=None) -> None:
    mn = _mn(M, N)
    _check("rmsnorm_fwd_residual",
           lib.rmsnorm_fwd_residual(_arg(x, "x", "act", dtype, mn), _arg(res, "res", "act", dtype, mn),
                                    _arg(w, "w", "weight", dtype, int(N)), float(eps), int(M), int(N), int(dtype),
                                    _arg(h, "h", "act", dtype, mn), _arg(y, "y", "act", dtype, mn),
                                    _arg(rstd, "rstd", "f32", count=int(M)),
                                    None if cfg is None else ctypes.byref(cfg), _stream(stream)))


def rmsnorm_bwd_residual(h, w, dy, dh, rstd, M, N, dtype, dx, dw, workspace, workspace_bytes, cfg=None,
                         stream=None) -> None:
    mn = _mn(M, N)
    _check("rmsnorm_bwd_residual",
           lib.rmsnorm_bwd_residual(_arg(h, "h", "act", dtype, mn), _arg(w, "w", "weight", dtype, int(N)),
                                    _arg(dy, "dy", "act", dtype, mn), _arg(dh, "dh", "act", dtype, mn),
                                    _arg(rstd, "rstd", "f32", count=int(M)), int(M), int(N), int(dtype),
                                    _arg(dx, "dx", "act", dtype, mn), _arg(dw, "dw", "f32", count=int(N)),
                                    _arg(workspace, "workspace", nbytes=int(workspace_bytes)),
                                    int(workspace_bytes), None if cfg is None else ctypes.byref(cfg),
                                    _stream(stream)))


def rmsnorm_bwd_rows(x, w, dy, rstd, M, N, dtype, dx, workspace, workspace_bytes, stream=None) -> int:
    """Backward row kernel only; returns the number of partial dW rows written."""
    p = ctypes.c_int64(0)
    mn = _mn(M, N)
    _check("rmsnorm_bwd_rows", lib.rmsnorm_bwd_rows(_arg(x, "x", "act", dtype, mn),
                                                    _arg(w, "w", "weight", dtype, int(N)),
                                                    _arg(dy, "dy", "act", dtype, mn),
                                                    _arg(rstd, "rstd", "f32", count=int(M)), int(M), int(N),
                                                    int(dtype), _arg(dx, "dx", "act", dtype, mn),
                                                    _arg(workspace, "workspace", nbytes=int(workspace_bytes)),
                                                    int(workspace_bytes), ctypes.byref(p), _stream(stream)))
    return int(p.value)


def rmsnorm_bwd_combine(workspace, partial_rows, N, dw, stream=None) -> None:
    ldp = (int(N) + 63) // 64 * 64
    _check("rmsnorm_bwd_combine",
           lib.rmsnorm_bwd_combine(_arg(workspace, "workspace", nbytes=int(partial_rows) * ldp * 4),
                                   int(partial_rows), int(N), _arg(dw, "dw", "f32", count=int(N)), _stream(stream)))


def rmsnorm_select_config(M, N, dtype, is_bwd, aligned, num_cus, blocks_per_cu) -> rmsnorm_config:
    cfg = rmsnorm_config()
    _check("rmsnorm_select_config",
           lib.rmsnorm_select_config(int(M), int(N), int(dtype), int(is_bwd), int(aligned), int(num_cus),
                                     int(blocks_per_cu), ctypes.byref(cfg)))
    return cfg


def rmsnorm_query_config(M, N, dtype, is_bwd) -> rmsnorm_config:
    cfg = rmsnorm_config()
    _check("rmsnorm_query_config",
           lib.rmsnorm_query_config(int(M), int(N), int(dtype), int(is_bwd), ctypes.byref(cfg)))
    return cfg


def rmsn_probe_copy(src, dst, nbytes, grid=0, variant=0, stream=None) -> None:
    _check("rmsn_probe_copy", bench_lib().rmsn_probe_copy(_arg(src, "src", nbytes=int(nbytes)),
                                                  _arg(dst, "dst", nbytes=int(nbytes)), int(nbytes), int(grid),
                                                  int(variant), _stream(stream)))


def rmsn_probe_write(dst, nbytes, grid=0, variant=0, stream=None) -> None:
    _check("rmsn_probe_write", bench_lib().rmsn_probe_write(_arg(dst, "dst", nbytes=int(nbytes)), int(nbytes), int(grid),
                                                    int(variant), _stream(stream)))


def rmsn_probe_read(src, nbytes, sink, grid=0, variant=0, stream=None) -> None:
    _check("rmsn_probe_read", bench_lib().rmsn_probe_read(_arg(src, "src", nbytes=int(nbytes)), int(nbytes), int(grid),
                                                  int(variant), _arg(sink, "sink", nbytes=16), _stream(stream)))


def rmsn_probe_add(a, b, c, nbytes, grid=0, variant=0, stream=None) -> None:
    _check("rmsn_probe_add", bench_lib().rmsn_probe_add(_arg(a, "a", nbytes=int(nbytes)), _arg(b, "b", nbytes=int(nbytes)),
                                                _arg(c, "c", nbytes=int(nbytes)), int(nbytes), int(grid),
                                                int(variant), _stream(stream)))


def rmsn_unfused_fwd(x, w, eps, M, N, dtype, y, rstd, stream=None) -> None:
    mn = _mn(M, N)
    _check("rmsn_unfused_fwd", bench_lib().rmsn_unfused_fwd(_arg(x, "x", "act", dtype, mn),
                                                    _arg(w, "w", "weight", dtype, int(N)), float(eps), int(M),
                                                    int(N), int(dtype), _arg(y, "y", "act", dtype, mn),
                                                    _arg(rstd, "rstd", "f32", count=int(M)), _stream(stream)))


def rmsn_unfused_bwd_workspace_bytes(M, N, dtype) -> int:
    n = int(bench_lib().rmsn_unfused_bwd_workspace_bytes(int(M), int(N), int(dtype)))
    if n < 0:
        raise RmsnormError("rmsn_unfused_bwd_workspace_bytes", n, rmsnorm_status_str(n))
    return n


def rmsn_unfused_bwd(x, w, dy, rstd, M, N, dtype, dx, dw, workspace, workspace_bytes, stream=None) -> None:
    mn = _mn(M, N)
    _check("rmsn_unfused_bwd", bench_lib().rmsn_unfused_bwd(_arg(x, "x", "act", dtype, mn),
                                                    _arg(w, "w", "weight", dtype, int(N)),
                                                    _arg(dy, "dy", "act", dtype, mn),
                                                    _arg(rstd, "rstd", "f32", count=int(M)), int(M), int(N),
                                                    int(dtype), _arg(dx, "dx", "act", dtype, mn),
                                                    _arg(dw, "dw", "f32", count=int(N)),
                                                    _arg(workspace, "workspace", nbytes=int(workspace_bytes)),
                                                    int(workspace_bytes), _stream(stream)))


def rmsn_add(a, b, c, n, dtype, stream=None) -> None:
    _check("rmsn_add", bench_lib().rmsn_add(_arg(a, "a", "act", dtype, int(n)), _arg(b, "b", "act", dtype, int(n)),
                                    _arg(c, "c", "act", dtype, int(n)), int(n), int(dtype), _stream(stream)))
