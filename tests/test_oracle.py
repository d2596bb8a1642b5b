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


def test_input_preparation_maps():
    # the preparation maps against library routines and their defining
    # properties (torch's elu, numpy's logaddexp, scipy's expit)
    import numpy as np
    import scipy.special
    import torch
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 5, 16)) * 3
    l2 = oracle.prepare_qk(x, "l2")
    assert np.allclose(np.linalg.norm(l2, axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(l2 * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-13, atol=0)
    assert np.array_equal(oracle.prepare_qk(np.zeros((2, 4)), "l2"), np.zeros((2, 4)))
    e = oracle.prepare_qk(x, "elu1")
    assert np.allclose(e, torch.nn.functional.elu(torch.from_numpy(x)).numpy() + 1.0,
                       rtol=1e-14, atol=1e-15)
    assert np.all(e > 0)
    g = oracle.prepare_gate(x, "neg_softplus")
    assert np.allclose(g, -np.logaddexp(0.0, x), rtol=1e-14, atol=1e-15)
    assert np.all(g < 0) and abs(oracle.prepare_gate(np.zeros(1), "neg_softplus")[0] + np.log(2)) < 1e-15
    b = oracle.prepare_beta(x, "sigmoid")
    assert np.allclose(b, scipy.special.expit(x), rtol=1e-14, atol=1e-16)
    assert oracle.prepare_beta(np.zeros(1), "sigmoid")[0] == 0.5
    assert oracle.prepare_qk(x, "identity") is not None and np.array_equal(oracle.prepare_qk(x, "identity"), x)
