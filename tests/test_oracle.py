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


def test_chunk_backward_equals_oracle(orc):
    # the chunk-level backward equations the HIP backward runs (three passes:
    # incoming states, gradients of the outgoing states newest first, then
    # per-chunk gradients) equal the oracle's reverse-mode recurrence at any C
    import numpy as np
    from chunk_form import chunk_backward
    from pins import rand_case, rel_err
    rng = np.random.default_rng(19)
    B, H, T, dk, dv = 1, 1, 45, 6, 5
    for rule in ("add", "delta"):
        for gate in ("none", "scalar", "channel"):
            q, k, v, g, beta, S0 = rand_case(rng, B, H, T, dk, dv, gate=gate, gate_scale=0.5)
            do = rng.standard_normal((B, H, T, dv))
            dsT = rng.standard_normal((B, H, dk, dv))
            ref = orc.recurrence_bwd(q, k, v, g, beta, S0, do, dsT, rule=rule, gate=gate)
            for C in (1, 7, 16, 45):
                out = chunk_backward(q[0, 0], k[0, 0], v[0, 0], None if g is None else g[0, 0],
                                     beta[0, 0], S0[0, 0], do[0, 0], dsT[0, 0], rule=rule, gate=gate, C=C)
                for name, a in zip(("dq", "dk", "dv", "dg", "dbeta", "ds0"), out):
                    if ref[name] is None:
                        assert a is None
                        continue
                    assert rel_err(a, ref[name][0, 0]) < 1e-12, f"{name} ({rule}/{gate}, C={C})"
