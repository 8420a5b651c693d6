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

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "rmsnorm_oracle.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "librmsnorm_oracle.so")

_DTYPE_CODE = {"f32": 0, "bf16": 1, "f64": 2}
_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}


def build(source: str = SOURCE, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Werror",
           *extra_flags, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """Handle on one compiled copy of the oracle library."""

    def __init__(self, lib_path: str):
        self.path = lib_path
        lib = ctypes.CDLL(lib_path)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.rmsn_oracle_fwd.argtypes = [vp, vp, ctypes.c_int, i64, i64, dp, vp, i64, vp, vp]
        lib.rmsn_oracle_bwd_dx.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, dp, vp, i64, vp, vp]
        lib.rmsn_oracle_bwd_dw.argtypes = [vp, vp, ctypes.c_int, i64, i64, dp, vp]
        for f in (lib.rmsn_oracle_fwd, lib.rmsn_oracle_bwd_dx, lib.rmsn_oracle_bwd_dw):
            f.restype = ctypes.c_int
        self._lib = lib

    @staticmethod
    def _check(a, dtype, shape):
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

    def fwd(self, x, w, eps, dtype, rows=None, want_y=True):
        """Return (y, r) in float64 for the listed rows (all rows by default)."""
        M, N = np.shape(x)
        x = self._check(x, dtype, (M, N))
        w = self._check(w, dtype, (N,))
        rows_a, n = self._rows(rows, M)
        y = np.empty((n, N), dtype=np.float64) if want_y else None
        r = np.empty(n, dtype=np.float64)
        rc = self._lib.rmsn_oracle_fwd(
            x.ctypes.data, w.ctypes.data, _DTYPE_CODE[dtype], M, N, float(eps),
            None if rows_a is None else rows_a.ctypes.data, n,
            None if y is None else y.ctypes.data, r.ctypes.data)
        if rc != 0:
            raise ValueError("oracle forward rejected its arguments")
        return y, r

    def bwd_dx(self, x, w, dy, eps, dtype, rows=None):
        """Return (dx, r) in float64 for the listed rows (all rows by default)."""
        M, N = np.shape(x)
        x = self._check(x, dtype, (M, N))
        w = self._check(w, dtype, (N,))
        dy = self._check(dy, dtype, (M, N))
        rows_a, n = self._rows(rows, M)
        dx = np.empty((n, N), dtype=np.float64)
        r = np.empty(n, dtype=np.float64)
        rc = self._lib.rmsn_oracle_bwd_dx(
            x.ctypes.data, w.ctypes.data, dy.ctypes.data, _DTYPE_CODE[dtype], M, N,
            float(eps), None if rows_a is None else rows_a.ctypes.data, n,
            dx.ctypes.data, r.ctypes.data)
        if rc != 0:
            raise ValueError("oracle backward (dx) rejected its arguments")
        return dx, r

    def bwd_dw(self, x, dy, eps, dtype):
        """Return dW (float64, length N) summed over every row."""
        M, N = np.shape(x)
        x = self._check(x, dtype, (M, N))
        dy = self._check(dy, dtype, (M, N))
        dw = np.empty(N, dtype=np.float64)
        rc = self._lib.rmsn_oracle_bwd_dw(x.ctypes.data, dy.ctypes.data, _DTYPE_CODE[dtype],
                                          M, N, float(eps), dw.ctypes.data)
        if rc != 0:
            raise ValueError("oracle backward (dW) rejected its arguments")
        return dw


_default = None


def get() -> Oracle:
    """The oracle built from ``rmsnorm_oracle.c`` (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def fwd(x, w, eps, dtype, rows=None, want_y=True):
    return get().fwd(x, w, eps, dtype, rows=rows, want_y=want_y)


def bwd_dx(x, w, dy, eps, dtype, rows=None):
    return get().bwd_dx(x, w, dy, eps, dtype, rows=rows)


def bwd_dw(x, dy, eps, dtype):
    return get().bwd_dw(x, dy, eps, dtype)
