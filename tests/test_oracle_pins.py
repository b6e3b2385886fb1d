"""The CPU oracle against its pins (closed forms, the pages' printed sizes,
torch's float64 attention, and the invariants the pages state)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(lib, pin):
    pin(lib)


def test_oracle_rejects_bad_arguments(lib):
    import numpy as np
    kc = np.zeros((1, 1, 2, 4, 4), np.float32)
    q = np.zeros((1, 1, 3, 1, 4), np.float32)  # 3 query heads over 2 KV heads
    with pytest.raises(oracle.OracleError):
        oracle.attention(q, kc, kc.copy(), np.zeros(1, np.int32), 1.0, lib=lib)
    q = np.zeros((1, 1, 2, 1, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.attention(q, kc, kc.copy(), np.array([4], np.int32), 1.0, lib=lib)


def test_oracle_empty_calls_are_noops(lib):
    import numpy as np
    kc = np.zeros((1, 1, 2, 4, 4), np.float32)
    kn = np.zeros((1, 1, 2, 0, 4), np.float32)
    oracle.append(kc, kc.copy(), kn, kn, np.array([4], np.int32), lib=lib)
    q = np.zeros((1, 1, 2, 0, 4), np.float32)
    out = oracle.attention(q, kc, kc.copy(), np.array([4], np.int32), 1.0, lib=lib)
    assert out.size == 0
