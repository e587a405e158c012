"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_errors(orc):
    import numpy as np
    dct = np.zeros((1, 2, 3), np.int32)
    diag = np.ones((1, 1, 4, 3), np.float32)
    sel = np.array([[[0, 1, 2, 0]]], np.int32)          # 2 is out of range for K=2
    with pytest.raises(ValueError, match="selection"):
        orc.scan(sel, "sel_i32", dct, diag, diag, diag, complex=False, bc_bf16=False)
    dct[0, 1, 2] = 3                                     # map entry out of range for N=3
    sel[0, 0, 2] = 1
    with pytest.raises(ValueError, match="map"):
        orc.scan(sel, "sel_i32", dct, diag, diag, diag, complex=False, bc_bf16=False)
