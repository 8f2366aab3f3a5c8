"""CPU pins of the float64 oracle (brute force, closed forms, invariants, formats)."""
import numpy as np
import pytest

import oracle.mla_oracle as O
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()


def test_empty_visible_set_convention():
    """Reading (parity unpinned): a query that sees no key yields zeros and lse = -inf."""
    q = np.ones((1, 2, 576))
    cache = np.ones((1, 4, 576))
    table = np.array([[0]], dtype=np.int32)
    out, lse = O.decode_paged_f64(q, np.array([0, 1], np.uint32), table, np.array([0], np.int32),
                                  cache, 4, 0.1, "causal")
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_visible_range_examples():
    # causal decode, one token: all L keys; three tokens: positions L-3, L-2, L-1
    assert O.visible_range(10, 1, 0, "causal") == (0, 10)
    assert [O.visible_range(10, 3, j, "causal") for j in range(3)] == [(0, 8), (0, 9), (0, 10)]
    assert O.visible_range(10, 3, 0, "null") == (0, 10)
    assert O.visible_range(10, 1, 0, "sliding_window_causal", 4) == (6, 10)
    with pytest.raises(ValueError):
        O.visible_range(10, 1, 0, "bogus")
