"""Pins of the second-order routing score (oracle/taylor.py), CPU only."""
import math

import numpy as np
import pytest

from oracle import sla, taylor

rng = np.random.default_rng(13)


def test_block_variance_closed_forms():
    n, d, block = 40, 5, 8
    x = np.repeat(rng.standard_normal((5, d)), block, axis=0)       # constant blocks
    np.testing.assert_allclose(taylor.block_variance(x, block), 0.0, atol=1e-28)
    y = np.zeros((n, d))
    y[:, 2] = np.tile([3.0, -3.0], n // 2)                          # +-c alternately
    v = taylor.block_variance(y + 7.0, block)
    np.testing.assert_allclose(v[:, 2], 9.0, rtol=1e-14)
    np.testing.assert_allclose(np.delete(v, 2, axis=1), 0.0, atol=1e-14)


def test_block_variance_brute_force_with_short_tail():
    n, d, block = 29, 3, 8
    x = rng.standard_normal((n, d))
    v = taylor.block_variance(x, block)
    for j, (a, b) in enumerate(sla.block_ranges(n, block)):
        for c in range(d):
            vals = [x[t, c] for t in range(a, b)]
            m = sum(vals) / len(vals)
            want = sum((u - m) ** 2 for u in vals) / len(vals)
            assert abs(v[j, c] - want) <= 1e-13


def test_zero_variance_gives_the_sla_route():
    n, d, block = 64 * 12, 16, 64
    q = rng.standard_normal((n, d))
    k = np.repeat(rng.standard_normal((12, d)), block, axis=0)
    a = taylor.route_taylor(q, k, 3, 4)
    b = sla.route(q, k, 3, 4)
    np.testing.assert_array_equal(a["logits"], b["logits"])
    np.testing.assert_array_equal(a["crit_idx"], b["crit_idx"])
    np.testing.assert_array_equal(a["marg_idx"], b["marg_idx"])


@pytest.mark.parametrize("eps", [1e-2, 3e-3])
def test_score_matches_block_mass_to_fourth_order(eps):
    # tokens come in +-c pairs along one feature each, so the block
    # covariance is exactly diagonal and the odd terms of the expansion
    # cancel: log mean_n exp(q' . k_n) differs from the second-order score by
    # at most about x^4 / 24 with x = max_n |q' . (k_n - kbar)| (the cosh
    # series remainder; x^4 / 12 leaves room), while the second-order term
    # itself (what the SLA logit misses) is of order eps^2
    d = 8
    kbar = rng.standard_normal(d)
    dev = []
    for rep in (1.0, 2.5):
        for a in range(d):
            for sgn in (1.0, -1.0):
                e = np.zeros(d)
                e[a] = sgn * eps * rep * (1 + a % 3)
                dev.append(e)
    dev = np.array(dev)
    k = kbar + dev
    n = k.shape[0]
    qbar = rng.standard_normal(d) * 2.0
    s = taylor.taylor_logits(qbar[None], k.mean(axis=0)[None], taylor.block_variance(k, n))[0, 0]
    exact = np.log(np.mean(np.exp(k @ qbar / math.sqrt(d))))
    x = np.abs(dev @ qbar / math.sqrt(d)).max()
    sla_logit = qbar @ kbar / math.sqrt(d)
    assert abs(s - exact) <= x ** 4 / 12, (s, exact, x)
    assert abs(sla_logit - exact) > 10 * x ** 4 / 12


def test_more_spread_more_score():
    d = 6
    qp = rng.standard_normal((3, d))
    kp = rng.standard_normal((4, d))
    kv = rng.uniform(0.1, 1.0, (4, d))
    base = taylor.taylor_logits(qp, kp, kv)
    kv2 = kv.copy()
    kv2[2] *= 1.5
    more = taylor.taylor_logits(qp, kp, kv2)
    assert np.all(more[:, 2] > base[:, 2])
    np.testing.assert_array_equal(np.delete(more, 2, axis=1), np.delete(base, 2, axis=1))


def test_logits_brute_force():
    d = 5
    qp = rng.standard_normal((3, d))
    kp = rng.standard_normal((4, d))
    kv = rng.uniform(0.0, 2.0, (4, d))
    got = taylor.taylor_logits(qp, kp, kv)
    for i in range(3):
        for j in range(4):
            first = sum(qp[i, a] * kp[j, a] for a in range(d)) / math.sqrt(d)
            second = sum(qp[i, a] ** 2 * kv[j, a] for a in range(d)) / (2 * d)
            assert abs(got[i, j] - (first + math.log(1 + second))) <= 1e-13
