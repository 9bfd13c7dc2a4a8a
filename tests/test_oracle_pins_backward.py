"""Pins of the backward pass (oracle/backward.py), CPU only.

Every gradient is checked against central finite differences of the
forward (oracle/sla.py) on tiny inputs: the forward and the finite
differences share no arithmetic with the chain-rule code.
"""
import numpy as np
import pytest

from oracle import backward as bwd
from oracle import sla

rng = np.random.default_rng(23)


def _lists(nb, kc, km, r):
    crit, marg = [], []
    for _ in range(nb):
        perm = r.permutation(nb)
        crit.append(np.sort(perm[:kc]))
        marg.append(np.sort(perm[kc:kc + km]))
    return np.array(crit, dtype=np.int64).reshape(nb, kc), np.array(marg, dtype=np.int64).reshape(nb, km)


def _loss(q, k, v, crit, marg, alpha, do, block):
    H, z = sla.linear_states(k, v, block)
    o, _, _ = sla.forward_head(q, k, v, crit, marg, H, z, alpha, block)
    return float((o * do).sum())


def _fd(fn, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        e = it.multi_index
        old = x[e]
        x[e] = old + h
        lp = fn()
        x[e] = old - h
        lm = fn()
        x[e] = old
        g[e] = (lp - lm) / (2 * h)
    return g


@pytest.mark.parametrize("n,kc,km,alpha", [(20, 1, 1, 0.6), (21, 2, 1, 0.3), (24, 0, 2, 0.5),
                                           (17, 3, 0, 0.7)])
def test_gradients_match_finite_differences(n, kc, km, alpha):
    d, block = 4, 8
    nb = -(-n // block)
    r = np.random.default_rng(n + kc)
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    do = r.standard_normal((n, d))
    crit, marg = _lists(nb, kc, km, r)
    dq, dk, dv, da = bwd.backward_head(q, k, v, crit, marg, alpha, do, block)
    f = lambda: _loss(q, k, v, crit, marg, alpha, do, block)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        np.testing.assert_allclose(g, _fd(f, x), rtol=1e-6, atol=1e-7)
    h = 1e-6
    fa = (_loss(q, k, v, crit, marg, alpha + h, do, block)
          - _loss(q, k, v, crit, marg, alpha - h, do, block)) / (2 * h)
    assert abs(da - fa) < 1e-7 * max(1.0, abs(fa))


def test_alpha_endpoints_isolate_the_branches():
    n, d, block = 24, 4, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    crit, marg = _lists(3, 1, 1, rng)
    dq1, dk1, dv1, _ = bwd.backward_head(q, k, v, crit, marg, 1.0, do, block)
    s = bwd.sparse_branch_backward(q, k, v, crit, do, block)
    for a, b in zip((dq1, dk1, dv1), s):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    dq0, dk0, dv0, _ = bwd.backward_head(q, k, v, crit, marg, 0.0, do, block)
    lb = bwd.linear_branch_backward(q, k, v, marg, do, block)
    for a, b in zip((dq0, dk0, dv0), lb):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_phi_backward_annihilates_constant_shifts():
    # phi(x + c 1) = phi(x), so a gradient along 1 has no effect: the input
    # gradient of any upstream gradient sums to zero per row
    x = rng.standard_normal((5, 7))
    f = sla.phi(x)
    g = bwd.phi_backward(f, rng.standard_normal((5, 7)))
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose(bwd.phi_backward(f, np.ones((5, 7)) * 3.0), 0.0, atol=1e-14)


def test_all_critical_dense_gradients():
    # every block critical: dense softmax attention, whose Q gradient has the
    # textbook closed form written here directly
    n, d = 16, 4
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    crit = np.tile(np.arange(2), (2, 1))
    dq, dk, dv = bwd.sparse_branch_backward(q, k, v, crit, do, 8)
    s = q @ k.T / 2.0
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dvt = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    np.testing.assert_allclose(dv, dvt, rtol=1e-12)
    np.testing.assert_allclose(dq, ds @ k / 2.0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk, ds.T @ q / 2.0, rtol=1e-12, atol=1e-14)
