"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_invalid_arguments_rejected(orc):
    import numpy as np
    q = np.zeros((1, 1, 0, 4))
    with pytest.raises(RuntimeError):
        orc.attn_fwd(q, q, q, 1.0, False)
    q = np.zeros((4, 2))
    with pytest.raises(RuntimeError):
        orc.attn_rows(q, q, q, 1.0, False, [4])
