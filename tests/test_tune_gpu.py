"""The configuration search on the GPU: the winner is a valid configuration whose
results match the oracle, and the cache returns it without re-timing."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import memory_bound_normalization_rmsnorm_amd as rn  # noqa: E402
from memory_bound_normalization_rmsnorm_amd import tune  # noqa: E402
import oracle  # noqa: E402
import synthetic_inputs as si  # noqa: E402
from parity_util import check_dw, check_rows, check_rstd, gpu_bwd, gpu_fwd, term_rms  # noqa: E402


@pytest.mark.parametrize("is_bwd", [0, 1])
@pytest.mark.parametrize("M,N", [(2048, 1024), (1000, 4100),   # 4100: the element kernels
                                 (64, 65536), (16, 262144)])   # split rows; the two-pass forward
def test_tuned_config_is_correct_and_cached(is_bwd, M, N, tmp_path):
    dtype = "bf16"
    print(f"tune M={M} N={N} is_bwd={is_bwd}", flush=True)
    path = str(tmp_path / "tuned.json")
    cfg = tune.best_config(M, N, rn.BF16, is_bwd, cache_path=path, budget_s=5.0)
    entry = next(iter(tune.load_cache(path).values()))
    assert entry["us"] <= entry["default_us"] * 1.0001 and entry["candidates_timed"] >= 1
    again = tune.best_config(M, N, rn.BF16, is_bwd, cache_path=path, budget_s=0.0)
    assert tune._key(again) == tune._key(cfg)
    x, w, dy = si.random_case(M, N, dtype, seed=31, dy_scale=1e-2)
    eps = si.eps_f32(1e-6)
    if is_bwd:
        _, rstd = gpu_fwd(x, w, eps, dtype)
        dx, dw = gpu_bwd(x, w, dy, rstd, dtype, cfg=cfg)
        odx, orr = oracle.bwd_dx(x, w, dy, eps, dtype)
        check_rows(dx, odx, dtype, "dx", floor=term_rms(x, w, dy, orr, dtype))
        check_dw(dw, oracle.bwd_dw(x, dy, eps, dtype), dtype)
    else:
        y, rstd = gpu_fwd(x, w, eps, dtype, cfg=cfg)
        oy, orr = oracle.fwd(x, w, eps, dtype)
        check_rows(y, oy, dtype, "y")
        check_rstd(rstd, orr)
    assert np.all(np.isfinite(rstd))
