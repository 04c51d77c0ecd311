"""The oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_golden_fixture_counts():
    # every dtype has several hand-built blocks, each a full block
    for name, n in (("Q8_0", 3), ("Q4_0", 3), ("Q4_K", 4), ("Q6_K", 4)):
        assert len(pins.load_golden(name)) == n


def test_rejects_bad_shapes():
    blob = np.zeros(18 * 4, np.uint8)
    with pytest.raises(ValueError):
        oracle.matmul(oracle.Q4_0, blob, 2, 48, np.zeros((1, 48), np.float32))   # K % 32
    with pytest.raises(ValueError):
        oracle.matmul(99, blob, 2, 64, np.zeros((1, 64), np.float32))          # dtype
    with pytest.raises(ValueError):
        oracle.matmul(oracle.Q4_0, blob[:10], 2, 64, np.zeros((1, 64), np.float32))  # short blob


def test_zero_scale_gives_exact_zero():
    # S = 0 -> y = 0 exactly (a tolerance of tau*S demands it)
    blob = np.zeros(34 * 2, np.uint8)
    blob[2:34] = 5
    y, _, s = oracle.matmul(oracle.Q8_0, blob, 1, 64, np.ones((1, 64), np.float32))
    assert y[0, 0] == 0 and s[0, 0] == 0
