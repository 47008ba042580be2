"""The CPU oracle against its pins (golden fixtures, brute force, closed forms,
invariants).  CPU only."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin, lib):
    pin(lib)


def test_int32_topk_idx_is_widened(lib):
    import numpy as np
    idx = np.array([[1, 0], [-1, 1], [2, 1]], np.int32)
    a = oracle.layout(idx, 3, 2, 10, lib=lib)
    b = oracle.layout(idx.astype(np.int64), 3, 2, 10, lib=lib)
    assert a.dst.tolist() == b.dst.tolist()
