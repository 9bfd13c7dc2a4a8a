"""Pins of oracle/qat.py (the low-bit forward / 16-bit backward pairing)."""
import math

import numpy as np

from oracle import backward as obwd
from oracle import qat
from oracle import sla


def _case(n=200, d=16, seed=0, kc=2, km=1):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    r = sla.route(q, k, kc, km)
    crit, marg = r["crit_idx"], r["marg_idx"]
    do = rng.standard_normal((n, d))
    return q, k, v, crit, marg, do


def test_identity_quantiser_gives_the_exact_gradients():
    q, k, v, crit, marg, do = _case()
    got = qat.qat_backward_head(q, k, v, crit, marg, 0.6, do, quant=lambda x: x)
    ref = obwd.backward_head(q, k, v, crit, marg, 0.6, do)
    for a, b in zip(got[:3], ref[:3]):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    assert abs(got[3] - ref[3]) <= 1e-10 * max(1.0, abs(ref[3]))


def test_saved_statistics_of_the_exact_forward_give_the_plain_backward():
    q, k, v, crit, marg, do = _case(seed=1)
    o, lse = qat.sparse_forward_stats(q, k, v, crit)
    np.testing.assert_allclose(o, sla.sparse_branch(q, k, v, crit), rtol=1e-12, atol=1e-12)
    got = qat.sparse_branch_backward_saved(q, k, v, crit, do, o, lse)
    ref = obwd.sparse_branch_backward(q, k, v, crit, do)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_quantising_v_alone_moves_dq_dk_by_the_closed_form():
    q, k, v, crit, marg, do = _case(seed=2)
    vq = np.round(v * 4.0) / 4.0
    quant_v = lambda x: vq if x is v else x  # noqa: E731
    alpha = 1.0                                      # sparse branch only
    got = qat.qat_backward_head(q, k, v, crit, marg, alpha, do, quant=quant_v)
    ref = obwd.backward_head(q, k, v, crit, marg, alpha, do)
    np.testing.assert_allclose(got[2], ref[2], rtol=1e-10, atol=1e-12)   # dv exact
    n, d = q.shape
    o_exact = sla.sparse_branch(q, k, v, crit)
    o_q = sla.sparse_branch(q, k, vq, crit)
    shift = (do * (o_q - o_exact)).sum(axis=1)       # rowsum(dO_s * (O^q_s - O_s))
    ddq = np.zeros_like(q)
    ddk = np.zeros_like(k)
    for i, (a, b) in enumerate(sla.block_ranges(n)):
        toks = sla._block_tokens(crit[i], n, 64)
        s = q[a:b] @ k[toks].T / math.sqrt(d)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dsd = -p * shift[a:b, None]
        ddq[a:b] += dsd @ k[toks] / math.sqrt(d)
        ddk[toks] += dsd.T @ q[a:b] / math.sqrt(d)
    np.testing.assert_allclose(got[0] - ref[0], ddq, rtol=1e-8, atol=1e-10)
    np.testing.assert_allclose(got[1] - ref[1], ddk, rtol=1e-8, atol=1e-10)


def test_fp8_round_trip_is_the_quantiser_s_values():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((130, 8)).astype(np.float32)
    y = qat.fp8_round_trip(x)
    # within half a quantum of the scaled E4M3 grid: |y - x| <= 2^-4 |x| + tiny
    assert np.all(np.abs(y - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -9 * np.abs(x).max())
    assert not np.array_equal(y, x)
