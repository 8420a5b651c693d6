"""fp64 CPU oracle for RMSNorm forward and backward (ctypes wrapper).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library and
its Python binding never import it, and the two share no code.

The arithmetic lives in ``rmsnorm_oracle.c`` (plain C, double precision,
sums with the index ascending); see its header for the passages it follows.
Every function here only marshals numpy arrays to it.

Parity unpinned: none. Each entry point is pinned in ``tests/test_oracle.py``
by the pages' worked examples, closed forms, invariants, finite differences
and an independent library computation.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "rmsnorm_oracle.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "librmsnorm_oracle.so")

_DTYPE_CODE = {"f32": 0, "bf16": 1, "f64": 2, "f16": 3}
_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64, "f16": np.float16}


def build(source: str = SOURCE, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Werror",
           *extra_flags, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data


class Oracle:
    """Handle on one compiled copy of the oracle library."""

    def __init__(self, lib_path: str):
        self.path = lib_path
        lib = ctypes.CDLL(lib_path)
        i64, vp, dp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
        lib.rmsn_oracle_fwd.argtypes = [vp, vp, vp, ci, ci, i64, i64, dp, vp, i64, vp, vp, vp]
        lib.rmsn_oracle_bwd_dx.argtypes = [vp, vp, vp, vp, vp, ci, ci, i64, i64, dp, vp, i64, vp, vp]
        lib.rmsn_oracle_bwd_dw.argtypes = [vp, vp, vp, ci, i64, i64, dp, vp]
        lib.rmsn_oracle_round.argtypes = [vp, i64, ci, vp]
        for f in (lib.rmsn_oracle_fwd, lib.rmsn_oracle_bwd_dx, lib.rmsn_oracle_bwd_dw, lib.rmsn_oracle_round):
            f.restype = ctypes.c_int
        self._lib = lib

    @staticmethod
    def _check(a, dtype, shape):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype != _STORAGE[dtype]:
            raise TypeError(f"expected {_STORAGE[dtype]} storage for {dtype}, got {a.dtype}")
        if a.shape != shape:
            raise ValueError(f"expected shape {shape}, got {a.shape}")
        return a

    @staticmethod
    def _rows(rows, M):
        if rows is None:
            return None, M
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        return rows, rows.size

    def _fwd(self, x, res, w, eps, dtype, wdtype, rows, want_y):
        M, N = np.shape(x)
        wdtype = wdtype or dtype
        x = self._check(x, dtype, (M, N))
        res = self._check(res, dtype, (M, N))
        w = self._check(w, wdtype, (N,))
        rows_a, n = self._rows(rows, M)
        y = np.empty((n, N), dtype=np.float64) if want_y else None
        h = np.empty((n, N), dtype=np.float64) if res is not None else None
        r = np.empty(n, dtype=np.float64)
        rc = self._lib.rmsn_oracle_fwd(_ptr(x), _ptr(res), _ptr(w), _DTYPE_CODE[dtype], _DTYPE_CODE[wdtype],
                                       M, N, float(eps), _ptr(rows_a), n, _ptr(h), _ptr(y), r.ctypes.data)
        if rc != 0:
            raise ValueError("oracle forward rejected its arguments")
        return h, y, r

    def fwd(self, x, w, eps, dtype, rows=None, want_y=True, wdtype=None):
        """Return (y, r) in float64 for the listed rows (all rows by default)."""
        _, y, r = self._fwd(x, None, w, eps, dtype, wdtype, rows, want_y)
        return y, r

    def fwd_residual(self, x, res, w, eps, dtype, rows=None, want_y=True, wdtype=None):
        """Fused residual add: return (h, y, r), h = round(x + res) in `dtype`
        (as float64), y the forward of h."""
        return self._fwd(x, res, w, eps, dtype, wdtype, rows, want_y)

    def bwd_dx(self, x, w, dy, eps, dtype, rows=None, res=None, dh=None, wdtype=None):
        """Return (dx, r) in float64 for the listed rows (all rows by default).
        With res, the input is the stored sum round(x + res); dh is added to dx."""
        M, N = np.shape(x)
        wdtype = wdtype or dtype
        x = self._check(x, dtype, (M, N))
        res = self._check(res, dtype, (M, N))
        w = self._check(w, wdtype, (N,))
        dy = self._check(dy, dtype, (M, N))
        dh = self._check(dh, dtype, (M, N))
        rows_a, n = self._rows(rows, M)
        dx = np.empty((n, N), dtype=np.float64)
        r = np.empty(n, dtype=np.float64)
        rc = self._lib.rmsn_oracle_bwd_dx(_ptr(x), _ptr(res), _ptr(w), _ptr(dy), _ptr(dh), _DTYPE_CODE[dtype],
                                          _DTYPE_CODE[wdtype], M, N, float(eps), _ptr(rows_a), n,
                                          dx.ctypes.data, r.ctypes.data)
        if rc != 0:
            raise ValueError("oracle backward (dx) rejected its arguments")
        return dx, r

    def bwd_dw(self, x, dy, eps, dtype, res=None):
        """Return dW (float64, length N) summed over every row."""
        M, N = np.shape(x)
        x = self._check(x, dtype, (M, N))
        res = self._check(res, dtype, (M, N))
        dy = self._check(dy, dtype, (M, N))
        dw = np.empty(N, dtype=np.float64)
        rc = self._lib.rmsn_oracle_bwd_dw(_ptr(x), _ptr(res), _ptr(dy), _DTYPE_CODE[dtype], M, N, float(eps),
                                          dw.ctypes.data)
        if rc != 0:
            raise ValueError("oracle backward (dW) rejected its arguments")
        return dw

    def round(self, values, dtype):
        """Round float64 values to the storage format `dtype` (nearest, ties to even), as float64."""
        v = np.ascontiguousarray(values, dtype=np.float64)
        out = np.empty_like(v)
        if self._lib.rmsn_oracle_round(v.ctypes.data, v.size, _DTYPE_CODE[dtype], out.ctypes.data) != 0:
            raise ValueError("oracle rounding rejected its arguments")
        return out


_default = None
_lock = threading.Lock()


def get() -> Oracle:
    """The oracle built from ``rmsnorm_oracle.c`` (compiled on first use if
    absent). Thread-safe: the first callers of a process (for instance the
    worker threads of a row-blocked comparison) build and load it once."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
                build()
            _default = Oracle(LIB_PATH)
        return _default


def fwd(x, w, eps, dtype, rows=None, want_y=True, wdtype=None):
    return get().fwd(x, w, eps, dtype, rows=rows, want_y=want_y, wdtype=wdtype)


def fwd_residual(x, res, w, eps, dtype, rows=None, want_y=True, wdtype=None):
    return get().fwd_residual(x, res, w, eps, dtype, rows=rows, want_y=want_y, wdtype=wdtype)


def bwd_dx(x, w, dy, eps, dtype, rows=None, res=None, dh=None, wdtype=None):
    return get().bwd_dx(x, w, dy, eps, dtype, rows=rows, res=res, dh=dh, wdtype=wdtype)


def bwd_dw(x, dy, eps, dtype, res=None):
    return get().bwd_dw(x, dy, eps, dtype, res=res)


def round_to(values, dtype):
    return get().round(values, dtype)
