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
