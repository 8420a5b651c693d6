"""The fixed-order dW combine (rmsnorm_bwd_combine) on its own, through the
C ABI: partial rows written by the host, at shapes that select each slice
count the library picks (8, 16, 32 and 64 partial rows summed side by side,
chosen from the number of partial rows P and the width N), with ragged
widths. Every column against the fp64 sum of the same fp32 partial rows,
within half an fp32 ulp of the sum plus the bound of an fp64 sum of P terms
(the combine adds in fp64 and rounds once); and two calls bit-identical.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import memory_bound_normalization_rmsnorm_amd as rn  # noqa: E402
import synthetic_inputs as si  # noqa: E402

# (P, N): slices 8 (few rows, wide), 16, 32, 64 (narrow: launch-bound), ragged widths
CASES = [(32, 262144), (33, 262144 + 4), (64, 131072), (128, 65536 + 8), (256, 32768), (256, 32768 + 12),
         (256, 8192), (256, 4096), (512, 2048), (768, 128), (1, 5), (3, 1000), (200, 4100)]


@pytest.mark.parametrize("P,N", CASES, ids=lambda v: str(v))
def test_combine_sums_every_column(P, N):
    ldp = (N + 63) // 64 * 64
    part = si.random_tensor((P, ldp), "f32", seed=P * 7 + N).astype(np.float32)
    print(f"combine P={P} N={N}", flush=True)
    sys.stdout.flush()
    ws = torch.from_numpy(part).cuda()
    outs = []
    for _ in range(2):
        dw = torch.full((N,), float("nan"), device="cuda")
        rn.rmsnorm_bwd_combine(ws, P, N, dw)
        torch.cuda.synchronize()
        outs.append(dw.cpu().numpy())
    ref = part[:, :N].astype(np.float64).sum(axis=0)
    # the sums are fp64, rounded once to fp32: half an fp32 ulp of the sum plus
    # the fp64 accumulation's bound (an fp32 accumulation fails this on the
    # columns that cancel)
    bound = (2.0 ** -24) * np.abs(ref) + P * 2.0 ** -52 * np.abs(part[:, :N]).astype(np.float64).sum(axis=0) + 1e-300
    err = np.abs(outs[0].astype(np.float64) - ref)
    assert np.all(np.isfinite(outs[0])), "a column was not written"
    assert np.all(err <= bound), f"worst column {int(np.argmax(err / bound))}: {err.max()} > bound"
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), "two calls differ"
