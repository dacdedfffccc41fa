"""The oracle against its pins (closed forms, invariants, brute force, library
routines and hand-worked fixtures).  CPU only."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_thread_count_does_not_change_result(orc):
    import numpy as np
    from oracle_pins import rand_inputs
    q, k, v, g, beta, S0 = rand_inputs(np.random.default_rng(5), 1, 33, 6, 8, 8)
    o1, h1 = orc.forward(q, k, v, g, beta, h0=S0, n_threads=1)
    o4, h4 = orc.forward(q, k, v, g, beta, h0=S0, n_threads=4)
    assert (o1 == o4).all() and (h1 == h4).all()
