"""Seeded synthetic inputs for the RMSNorm workloads.

This module holds random-number generation and storage-format conversion
only (fp32 -> bf16 bit patterns by round-to-nearest-even, and back). None of
the normalisation arithmetic lives here. The fp64 CPU oracle and the GPU
library both read the arrays it returns, so the two sides always see
bit-identical inputs.

Storage conventions:
  * fp32 tensors are ``np.float32`` arrays;
  * bf16 tensors are ``np.uint16`` arrays holding the bf16 bit patterns;
  * fp16 tensors are ``np.float16`` arrays (numpy rounds to nearest even).

The workloads mirror the synthetic shapes measured on the pages: the Quack
Hopper study's widest row (32768 x 8192, "What a tuned RMSNorm kernel actually
costs on Hopper", sections 04-05), the QK-norm use mentioned on the
"RMSNorm backward (almost) without the column reduction" page (introduction),
and the fp32 1024 x 4096 regime of the hello-gpu chapter 13 (section 13.5).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DTYPES = ("f32", "bf16", "f16")


def f32_to_bf16_bits(a: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round finite fp32 values to bf16 (round-to-nearest-even) bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("synthetic inputs must be finite")
    u = a.reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    for s in range(0, u.size, chunk):
        c = u[s:s + chunk]
        # keep the high half; add 0x7FFF plus the lowest kept bit so that ties
        # go to even. No overflow for finite inputs (max 0xFF7FFFFF + 0x8000).
        out[s:s + chunk] = ((c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1)))
                            >> np.uint32(16)).astype(np.uint16)
    return out.reshape(a.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "f16":
        return np.ascontiguousarray(np.asarray(a32, dtype=np.float32).astype(np.float16))
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def eps_f32(eps: float) -> float:
    """The epsilon both sides use: the fp32 value nearest ``eps``, as a Python float."""
    return float(np.float32(eps))


@dataclass(frozen=True)
class Workload:
    """One synthetic RMSNorm workload (shape, dtype, epsilon and distributions)."""

    name: str
    dtype: str
    M: int
    N: int
    eps: float
    w_dist: str          # "normal" -> 1 + 0.1 N(0,1); "uniform" -> U(0.5, 1.5)
    dy_scale: float      # dy = dy_scale * N(0,1)
    seed: int            # x, w, dy use seed+1, seed+2, seed+3; outliers seed+4
    outlier_rows: int = 0
    outlier_cols: int = 0
    outlier_scale: float = 1.0
    description: str = ""

    def fwd_bytes(self) -> int:
        """Algorithmic bytes of one forward call: read x, w; write y, rstd."""
        s = 4 if self.dtype == "f32" else 2
        return 2 * self.M * self.N * s + self.N * s + 4 * self.M

    def bwd_bytes(self) -> int:
        """Algorithmic bytes of one backward call: read x, dy, w, rstd; write dx, dW."""
        s = 4 if self.dtype == "f32" else 2
        return 3 * self.M * self.N * s + self.N * s + 4 * self.M + 4 * self.N


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fp32_256x1024", "f32", 256, 1024, 1e-5, "normal", 1.0, 100,
                 description="fp32 256x1024, eps 1e-5; x~N(0,1), w=1+0.1N(0,1), dy~N(0,1)"),
        Workload("bf16_16384x4096", "bf16", 16384, 4096, 1e-6, "normal", 1e-2, 200,
                 description="bf16 16384x4096, eps 1e-6; x~N(0,1), w=1+0.1N(0,1), dy~1e-2 N(0,1)"),
        Workload("bf16_32768x8192_outliers", "bf16", 32768, 8192, 1e-6, "uniform", 1e-2, 300,
                 outlier_rows=16, outlier_cols=4, outlier_scale=50.0,
                 description="bf16 32768x8192, eps 1e-6; x~N(0,1) with 16 whole rows and 4 whole "
                             "columns scaled by 50 (0.098% of entries), w~U(0.5,1.5), dy~1e-2 N(0,1)"),
        Workload("bf16_qknorm_1048576x128", "bf16", 1048576, 128, 1e-6, "normal", 1e-2, 400,
                 description="QK-norm: 8 seqs x 4096 tokens x 32 heads = 1048576 rows of 128, bf16, "
                             "eps 1e-6; x~N(0,1), w=1+0.1N(0,1), dy~1e-2 N(0,1)"),
        Workload("bf16_4096x32768", "bf16", 4096, 32768, 1e-5, "uniform", 1e-2, 500,
                 description="wide row bf16 4096x32768, eps 1e-5; x~N(0,1), w~U(0.5,1.5), dy~1e-2 N(0,1)"),
        Workload("bf16_16384x5120", "bf16", 16384, 5120, 1e-5, "uniform", 1e-2, 510,
                 description="bf16 16384x5120, eps 1e-5; x~N(0,1), w~U(0.5,1.5), dy~1e-2 N(0,1)"),
        Workload("bf16_16384x7168", "bf16", 16384, 7168, 1e-5, "uniform", 1e-2, 520,
                 description="bf16 16384x7168, eps 1e-5; x~N(0,1), w~U(0.5,1.5), dy~1e-2 N(0,1)"),
        Workload("bf16_16384x4100", "bf16", 16384, 4100, 1e-5, "uniform", 1e-2, 530,
                 description="bf16 16384x4100 (8200-byte rows, not a multiple of 16 bytes), eps 1e-5; "
                             "x~N(0,1), w~U(0.5,1.5), dy~1e-2 N(0,1)"),
    ]
}


# Rows wider than one workgroup holds (the backward's split rows, the forward's
# 16 vectors per lane and its two-pass kernel): benchmarked and profiled with
# `bench.py --workload`, and checked at full size, beside the workloads above.
WIDE_WORKLOADS = {
    w.name: w
    for w in [
        Workload("bf16_4096x65536", "bf16", 4096, 65536, 1e-5, "uniform", 1e-2, 540,
                 description="wide row bf16 4096x65536, eps 1e-5; x~N(0,1), w~U(0.5,1.5), dy~1e-2 N(0,1)"),
        Workload("bf16_1024x262144", "bf16", 1024, 262144, 1e-5, "uniform", 1e-2, 550,
                 description="wide row bf16 1024x262144, eps 1e-5; x~N(0,1), w~U(0.5,1.5), dy~1e-2 N(0,1)"),
    ]
}


def workload(name: str) -> Workload:
    """A workload of WORKLOADS or WIDE_WORKLOADS by name."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    return WIDE_WORKLOADS[name]


def _normal_f32(seed: int, shape) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape, dtype=np.float32)


def make_x(wl: Workload) -> np.ndarray:
    x = _normal_f32(wl.seed + 1, (wl.M, wl.N))
    if wl.outlier_rows or wl.outlier_cols:
        rows, cols = outlier_picks(wl)
        is_row = np.zeros(wl.M, dtype=bool)
        is_row[rows] = True
        x[rows, :] *= np.float32(wl.outlier_scale)
        # columns: scale once, skipping entries already scaled as part of a row
        sub = x[~is_row][:, cols] * np.float32(wl.outlier_scale)
        x[np.ix_(np.nonzero(~is_row)[0], cols)] = sub
    return to_storage(x, wl.dtype)


def outlier_picks(wl: Workload):
    rng = np.random.Generator(np.random.PCG64(wl.seed + 4))
    rows = np.sort(rng.choice(wl.M, size=wl.outlier_rows, replace=False))
    cols = np.sort(rng.choice(wl.N, size=wl.outlier_cols, replace=False))
    return rows, cols


def make_w(wl: Workload) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(wl.seed + 2))
    if wl.w_dist == "normal":
        w = np.float32(1.0) + np.float32(0.1) * rng.standard_normal(wl.N, dtype=np.float32)
    elif wl.w_dist == "uniform":
        w = rng.uniform(0.5, 1.5, wl.N).astype(np.float32)
    else:
        raise ValueError(wl.w_dist)
    return to_storage(w, wl.dtype)


def make_dy(wl: Workload) -> np.ndarray:
    dy = _normal_f32(wl.seed + 3, (wl.M, wl.N))
    if wl.dy_scale != 1.0:
        dy *= np.float32(wl.dy_scale)
    return to_storage(dy, wl.dtype)


def make_inputs(wl: Workload):
    """Return (x, w, dy) in storage format for workload ``wl``."""
    return make_x(wl), make_w(wl), make_dy(wl)


def random_case(M: int, N: int, dtype: str, seed: int, x_scale: float = 1.0,
                dy_scale: float = 1.0, w_dist: str = "normal", wdtype: str | None = None):
    """Small seeded case for parity tests: (x, w, dy) in storage format (w in
    `wdtype`, default the activation format)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, N), dtype=np.float32) * np.float32(x_scale)
    if w_dist == "normal":
        w = np.float32(1.0) + np.float32(0.1) * rng.standard_normal(N, dtype=np.float32)
    else:
        w = rng.uniform(0.5, 1.5, N).astype(np.float32)
    dy = rng.standard_normal((M, N), dtype=np.float32) * np.float32(dy_scale)
    return to_storage(x, dtype), to_storage(w, wdtype or dtype), to_storage(dy, dtype)


def random_tensor(shape, dtype: str, seed: int, scale: float = 1.0) -> np.ndarray:
    """A seeded N(0, scale^2) tensor in storage format (residuals, gradients)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return to_storage(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale), dtype)
