"""The CPU oracle against facts fixed outside it (see tests/_pins.py)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle.pi_oracle as O

from . import _pins


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.booleans(), min_size=1, max_size=300))
def test_compaction_property(bits):
    _pins.check_compaction(O, np.array(bits, dtype=bool))


@settings(max_examples=50, deadline=None)
@given(st.integers(1, 8), st.integers(1, 120), st.integers(0, 2**31 - 1))
def test_union_property(B, F, seed):
    m = np.random.default_rng(seed).random((B, F)) < 0.2
    u = O.compact(O.union_active(m))
    want = sorted(set(int(i) for t in range(B) for i in np.flatnonzero(m[t])))
    assert list(u) == want
