"""The fp64 oracle against its pins (closed forms, invariants, brute force,
the pages' worked examples).  CPU only."""
import pytest

import oracle
from pins import PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_thread_count_does_not_change_result(orc):
    import numpy as np
    from pins import rand_case
    rng = np.random.default_rng(7)
    q, k, v, g, beta, s0 = rand_case(rng, 3, 3, 20, 4, 4, gate="channel")
    a = orc.recurrence(q, k, v, g, beta, s0, rule="delta", gate="channel", nthreads=1)
    b = orc.recurrence(q, k, v, g, beta, s0, rule="delta", gate="channel", nthreads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_bad_arguments(orc):
    import numpy as np
    q = np.zeros((1, 1, 4, 3))
    with pytest.raises(ValueError):
        orc.recurrence(q, q, q, None, None, None, rule="delta", gate="none")
    with pytest.raises(ValueError):
        orc.recurrence(q, q, q, np.zeros((1, 1, 4)), None, None, rule="add", gate="channel")
