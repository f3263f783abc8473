"""The CPU oracle against its pins (no GPU needed)."""
import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle)


def test_panels_change_nothing():
    """Row panels are a memory device only: rows never interact."""
    r = np.random.default_rng(3)
    q, k, v = (r.standard_normal((1, 2, 50, 8)) for _ in range(3))
    for causal in (False, True):
        o1, l1 = oracle.attention_forward(q, k, v, 0.3, causal, panel_rows=7)
        o2, l2 = oracle.attention_forward(q, k, v, 0.3, causal, panel_rows=4096)
        assert np.allclose(o1, o2, atol=1e-13, rtol=0) and np.allclose(l1, l2, atol=1e-13, rtol=0)


def test_row_samplers_match_full():
    r = np.random.default_rng(4)
    q, k, v, do = (r.standard_normal((2, 2, 40, 8)) for _ in range(4))
    rows = [0, 5, 39]
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, 0.3, causal)
        so, sl = oracle.attention_forward_rows(q, k, v, 0.3, causal, 1, 1, rows)
        assert np.allclose(so, o[1, 1, rows], atol=1e-13, rtol=0)
        assert np.allclose(sl, lse[1, 1, rows], atol=1e-13, rtol=0)
        for r0, r1 in ((0, 40), (0, 1), (17, 31), (39, 40)):
            po, pl = oracle.attention_forward_panel(q, k, v, 0.3, causal, 0, 1, r0, r1)
            assert np.allclose(po, o[0, 1, r0:r1], atol=1e-13, rtol=0)
            assert np.allclose(pl, lse[0, 1, r0:r1], atol=1e-13, rtol=0)
        dq, _, _ = oracle.attention_backward(q, k, v, do, 0.3, causal)
        sdq = oracle.attention_backward_rows(q, k, v, do, 0.3, causal, 1, 0, rows)
        assert np.allclose(sdq, dq[1, 0, rows], atol=1e-13, rtol=0)
        part = oracle.attention_backward(q, k, v, do, 0.3, causal, heads=[(0, 1)])
        assert np.allclose(part[(0, 1)][0], dq[0, 1], atol=0, rtol=0)


def test_backward_terms_give_the_gradients():
    """The exposed intermediates are the ones the gradients are built from:
    dV = P^T dO, dQ = scale dS K, dK = scale dS^T Q, D = rowsum(dO * O), and
    every dS row sums to zero."""
    r = np.random.default_rng(5)
    q, k, v, do = (r.standard_normal((1, 2, 23, 8)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.4, causal)
        o, _ = oracle.attention_forward(q, k, v, 0.4, causal)
        p, dp, dd, ds = oracle.attention_backward_terms(q, k, v, do, 0.4, causal, 0, 1)
        assert np.allclose(p.T @ do[0, 1], dv[0, 1], atol=1e-13, rtol=0)
        assert np.allclose(0.4 * ds @ k[0, 1], dq[0, 1], atol=1e-13, rtol=0)
        assert np.allclose(0.4 * ds.T @ q[0, 1], dk[0, 1], atol=1e-13, rtol=0)
        assert np.allclose(dp, do[0, 1] @ v[0, 1].T, atol=1e-13, rtol=0)
        assert np.allclose(dd, np.sum(do[0, 1] * o[0, 1], axis=1), atol=1e-12, rtol=0)
        assert np.allclose(ds.sum(axis=1), 0.0, atol=1e-12)
