"""The fp64 oracle against its pins (closed forms, invariants, libraries)."""
import pytest

from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_arguments(orc):
    import numpy as np
    q = np.zeros((1, 3, 8), np.float32)
    k = np.zeros((4, 2, 8), np.float32)
    with pytest.raises(ValueError):
        orc.attention(q, [0], k, k, 1.0)          # 3 % 2 != 0
    q = np.zeros((1, 2, 8), np.float32)
    with pytest.raises(ValueError):
        orc.attention(q, [4], k, k, 1.0)          # position past the slab
    with pytest.raises(ValueError):
        orc.attention(q, [-1], k, k, 1.0)
