"""The oracle against the facts that pin it (see tests/oracle_pins.py)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_rejects_bad_arguments(orc):
    import numpy as np

    K = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        orc.route(np.zeros((3, 5)), K, K, 1.0)  # D mismatch
    with pytest.raises(TypeError):
        orc.route(np.zeros((3, 2), np.float32), K, K, 1.0)  # mixed dtypes
