"""The fp64 oracle against facts outside itself (CPU only)."""
import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle.default())


def test_oracle_rejects_bad_arguments():
    import numpy as np
    z = np.zeros((2, 1, 2))
    with pytest.raises(ValueError):
        # slot beyond the pool
        oracle.prefill(z, z, z, z, np.zeros((2, 1)), [0, 2], np.zeros((1, 1, 2, 2)), [5])
    with pytest.raises(ValueError):
        # decreasing cu_seqlens
        oracle.prefill(z, z, z, z, np.zeros((2, 1)), [0, 2, 1], np.zeros((2, 1, 2, 2)), [0, 1])
