"""The fp64 oracle against its pins (no GPU).

Each pin checks the oracle against something other than itself: the printed
worked examples of hello-gpu chapter 13, closed forms, invariants, finite
differences and PyTorch's fp64 implementation. See ``oracle_pins.py``.
"""

import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.get())


def test_oracle_rejects_bad_arguments():
    x = np.ones((2, 3), np.float32)
    w = np.ones(3, np.float32)
    with pytest.raises(ValueError):
        oracle.fwd(x, w, -1.0, "f32")
    with pytest.raises(ValueError):
        oracle.fwd(x, w, float("nan"), "f32")
    with pytest.raises(ValueError):
        oracle.fwd(x, w, 1e-5, "f32", rows=[5])
    with pytest.raises(TypeError):
        oracle.fwd(x.astype(np.float64), w, 1e-5, "f32")


def test_oracle_empty_rows():
    x = np.zeros((0, 8), np.float32)
    w = np.ones(8, np.float32)
    y, r = oracle.fwd(x, w, 1e-5, "f32")
    assert y.shape == (0, 8) and r.shape == (0,)
    assert np.all(oracle.bwd_dw(x, x, 1e-5, "f32") == 0.0)


def test_oracle_row_blocks_match_one_call():
    """The blocked, threaded helper the full-size parity tests use returns the
    oracle's own rows, whatever the block size and thread split."""
    import numpy as np

    import synthetic_inputs as si
    from parity_util import oracle_row_blocks

    x, w, dy = si.random_case(37, 40, "bf16", seed=3, dy_scale=1e-2)
    oy, orr = oracle.fwd(x, w, 1e-6, "bf16")
    odx, _ = oracle.bwd_dx(x, w, dy, 1e-6, "bf16")
    for block, threads in ((8, 3), (37, 1), (100, 5)):
        got = list(oracle_row_blocks(x, w, dy, 1e-6, "bf16", block=block, threads=threads))
        assert sum(s.stop - s.start for s, *_ in got) == 37
        assert np.array_equal(np.concatenate([g[1] for g in got]), oy)
        assert np.array_equal(np.concatenate([g[2] for g in got]), orr)
        assert np.array_equal(np.concatenate([g[3] for g in got]), odx)
