"""The CPU oracle against its pins (closed forms, LTI identity, brute force, invariants)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(oracle_mod, pin):
    pin(oracle_mod)


def test_oracle_rejects_bad_arguments(oracle_mod):
    import numpy as np

    u = np.zeros((1, 4, 2), dtype=np.float32)
    A = -np.ones((2, 16), dtype=np.float32)
    Bm = np.zeros((1, 4, 16), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle_mod.scan(u, u, A, Bm[:, :3], Bm)
    with pytest.raises(ValueError):
        oracle_mod.scan(u, u, A, Bm, Bm, lanes=[2])          # lane out of range
    with pytest.raises(ValueError):
        oracle_mod.scan(u, u, A, Bm, Bm, record_t=[2, 1])    # not ascending
    with pytest.raises(TypeError):
        oracle_mod.scan(u.astype(np.float64), u, A, Bm, Bm)
