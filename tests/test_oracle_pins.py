"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
import oracle_pins



@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, lib):
    pin(lib)


def test_rejects_bad_shapes(lib):
    import numpy as np
    x = np.zeros(24, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.pack(x, 6, 1, 4, 1, 4, lib=lib)   # s % P != 0
    with pytest.raises(ValueError):
        oracle.pack(x, 4, 1, 6, 1, 4, lib=lib)   # h % P != 0
    q = np.zeros((4, 1, 3, 2), dtype=np.float32)
    k = np.zeros((4, 1, 2, 2), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.attn(q, k, k, 4, 1, 3, 2, 2, 1, False, lib=lib)  # h % h_kv != 0
