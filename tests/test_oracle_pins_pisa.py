"""Pins of piecewise exact-or-approximate attention (oracle/pisa.py), CPU only."""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import pisa, sla

rng = np.random.default_rng(17)


def _dense(q, k, v):
    """Textbook scaled dot-product softmax attention."""
    return softmax(q @ k.T / math.sqrt(q.shape[1]), axis=1) @ v


def _random_lists(nb, kc, rng_):
    return np.stack([np.sort(rng_.choice(nb, kc, replace=False)) for _ in range(nb)]) \
        if kc else np.zeros((nb, 0), dtype=np.int64)


def test_block_statistics_brute_force():
    n, d, dv, block = 21, 3, 2, 8
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, dv))
    kbar, vsum, cnt, H = pisa.block_statistics(k, v, block)
    starts = [0, 8, 16]
    for j, a in enumerate(starts):
        b = min(a + block, n)
        assert cnt[j] == b - a
        for f in range(d):
            mean = sum(k[t, f] for t in range(a, b)) / (b - a)
            assert abs(kbar[j, f] - mean) < 1e-14
            for c in range(dv):
                h = sum((k[t, f] - mean) * v[t, c] for t in range(a, b))
                assert abs(H[j, f, c] - h) < 1e-13
        for c in range(dv):
            assert abs(vsum[j, c] - sum(v[t, c] for t in range(a, b))) < 1e-13
    np.testing.assert_allclose(pisa.global_first_order(H), H.sum(axis=0) / 3, rtol=1e-14)


@pytest.mark.parametrize("n", [256, 250])
def test_nothing_unselected_is_dense_attention(n):
    d = 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    nb = -(-n // 64)
    crit = np.tile(np.arange(nb), (nb, 1))
    o, o_sm, o_fo = pisa.pisa_head(q, k, v, crit)
    np.testing.assert_allclose(o, _dense(q, k, v), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(o_fo, 0.0)


@pytest.mark.parametrize("n,kc", [(64 * 6, 0), (64 * 6, 2), (64 * 5 + 19, 1), (64 * 5 + 19, 3)])
def test_constant_key_blocks_make_the_expansion_exact(n, kc):
    # every key equals its block centroid: the zero-order terms are the
    # exact block contributions and every first-order matrix is 0, so the
    # result is dense attention whatever the selected set (the short last
    # block checks the token count in the denominator)
    d = 8
    nb = -(-n // 64)
    q = rng.standard_normal((n, d))
    k = np.repeat(rng.standard_normal((nb, d)) * 1.5, 64, axis=0)[:n]
    v = rng.standard_normal((n, 5))
    crit = _random_lists(nb, kc, rng)
    o, o_sm, o_fo = pisa.pisa_head(q, k, v, crit)
    np.testing.assert_allclose(o, _dense(q, k, v), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(o_fo, 0.0, atol=1e-13)


def _equal_first_order_case(eps, seed=3):
    # K = per-block centroid + eps * a mean-zero pattern shared by all blocks;
    # V = per-block offset + a pattern shared by all blocks.  Every block
    # then has the same first-order matrix, so the global correction is the
    # exact first-order term and the error left is of second order in eps.
    r = np.random.default_rng(seed)
    nb, d, dv = 6, 8, 4
    pat = r.standard_normal((64, d))
    pat -= pat.mean(axis=0)
    wpat = r.standard_normal((64, dv))
    k = (r.standard_normal((nb, 1, d)) + eps * pat[None]).reshape(nb * 64, d)
    v = (r.standard_normal((nb, 1, dv)) + wpat[None]).reshape(nb * 64, dv)
    q = r.standard_normal((nb * 64, d)) * 2.0
    crit = np.stack([np.sort(r.choice(nb, 2, replace=False)) for _ in range(nb)])
    o, o_sm, _ = pisa.pisa_head(q, k, v, crit)
    ref = _dense(q, k, v)
    return np.abs(o - ref).max(), np.abs(o_sm - ref).max()


def test_equal_first_order_matrices_leave_second_order_error():
    e1, z1 = _equal_first_order_case(0.02)
    e2, z2 = _equal_first_order_case(0.01)
    # with the correction: second order (halving eps quarters the error)
    assert 0.18 < e2 / e1 < 0.32, (e1, e2)
    # without it (zero order only): first order (halving eps halves it)
    assert 0.4 < z2 / z1 < 0.6, (z1, z2)
    assert e1 < 0.1 * z1


def test_brute_force_tiny():
    n, d, dv, block = 20, 3, 2, 8
    q = rng.standard_normal((n, d)) * 0.7
    k = rng.standard_normal((n, d)) * 0.7
    v = rng.standard_normal((n, dv))
    crit = np.array([[1], [0], [2]])
    o, _, _ = pisa.pisa_head(q, k, v, crit, block)
    blocks = [range(0, 8), range(8, 16), range(16, 20)]
    sq = math.sqrt(d)
    kb = [[sum(k[t, f] for t in blk) / len(blk) for f in range(d)] for blk in blocks]
    Hs = []
    for j, blk in enumerate(blocks):
        Hs.append([[sum((k[t, f] - kb[j][f]) * v[t, c] for t in blk) for c in range(dv)]
                   for f in range(d)])
    Hbar = [[sum(Hs[j][f][c] for j in range(3)) / 3 for c in range(dv)] for f in range(d)]
    for i, blk_i in enumerate(blocks):
        for t in blk_i:
            qt = [q[t, f] / sq for f in range(d)]
            num = [0.0] * dv
            den = 0.0
            asum = 0.0
            for j, blk in enumerate(blocks):
                if j in crit[i]:
                    for s in blk:
                        e = math.exp(sum(qt[f] * k[s, f] for f in range(d)))
                        den += e
                        for c in range(dv):
                            num[c] += e * v[s, c]
                else:
                    al = math.exp(sum(qt[f] * kb[j][f] for f in range(d)))
                    asum += al
                    den += al * len(blk)
                    for c in range(dv):
                        num[c] += al * sum(v[s, c] for s in blk)
            for c in range(dv):
                num[c] += asum * sum(qt[f] * Hbar[f][c] for f in range(d))
                assert abs(o[t, c] - num[c] / den) < 1e-12


def test_query_block_subset():
    n, d = 64 * 5 + 7, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    crit = _random_lists(6, 2, rng)
    full = pisa.pisa_head(q, k, v, crit)[0]
    part = pisa.pisa_head(q, k, v, crit, q_blocks=[1, 5])[0]
    rows = np.r_[64:128, 320:n]
    np.testing.assert_array_equal(part[rows], full[rows])
    other = np.setdiff1d(np.arange(n), rows)
    np.testing.assert_array_equal(part[other], 0.0)


# ---------------------------------------------------------------- covariance-aware routing

def test_block_deviation_brute_force_singular_values_and_spectral_bound():
    nb, d, dv = 5, 4, 3
    H = rng.standard_normal((nb, d, dv))
    Hbar = H.mean(axis=0)
    M = pisa.block_deviation(H, Hbar)
    for j in range(nb):
        ss = 0.0
        for a in range(d):
            for c in range(dv):
                ss += (H[j, a, c] - Hbar[a, c]) ** 2
        assert abs(M[j] - math.sqrt(ss)) < 1e-13
        sv = np.linalg.svd(H[j] - Hbar, compute_uv=False)
        assert abs(M[j] ** 2 - (sv ** 2).sum()) < 1e-12 * max(1.0, M[j] ** 2)
        assert M[j] >= sv[0] - 1e-13          # bounds the spectral norm ...
        for _ in range(20):                    # ... hence |q (H_j - Hbar)| <= |q| M_j
            qv = rng.standard_normal(d)
            assert np.linalg.norm(qv @ (H[j] - Hbar)) <= np.linalg.norm(qv) * M[j] + 1e-12
    np.testing.assert_array_equal(pisa.block_deviation(np.tile(H[:1], (nb, 1, 1)), H[0]), 0.0)


def test_covariance_logits_brute_force():
    nq, nkb, d = 3, 5, 8
    qp, kp = rng.standard_normal((nq, d)), rng.standard_normal((nkb, d))
    M = rng.uniform(0, 50, nkb)
    got = pisa.covariance_logits(qp, kp, M)
    for i in range(nq):
        qn = math.sqrt(sum(x * x for x in qp[i]))
        for j in range(nkb):
            s = sum(qp[i, a] * kp[j, a] for a in range(d)) / math.sqrt(d)
            want = s + math.log(1.0 + qn * M[j] / (math.sqrt(d) * 64))
            assert abs(got[i, j] - want) < 1e-12


def _signed_deviation_blocks(nb, d, n_last=64):
    # every block: the same centred key pattern Dk and values U + W or
    # U - W (half the blocks each), so H_j = Dk^T U +- Dk^T W, Hbar =
    # Dk^T U and every M_j is the same non-zero number while |H_j| is not;
    # the block means differ, so the plain logits do not tie
    n = 64 * (nb - 1) + n_last
    Dk = rng.standard_normal((64, d))
    Dk -= Dk.mean(axis=0)
    W = rng.standard_normal((64, d))
    U = 2.0 * rng.standard_normal((64, d))
    means = rng.standard_normal((nb, d))
    k = np.concatenate([means[j] + Dk for j in range(nb)])[:n]
    sign = np.array([1.0 if j % 2 == 0 else -1.0 for j in range(nb)])
    v = np.concatenate([U + sign[j] * W for j in range(nb)])[:n]
    q = rng.standard_normal((n, d))
    return q, k, v


def test_equal_deviations_give_the_plain_split():
    q, k, v = _signed_deviation_blocks(12, 16)
    r = pisa.route_pisa(q, k, v, 3, 4)
    M = r["block_dev"]
    assert M.min() > 1.0 and np.ptp(M) < 1e-9 * M.max()
    p = sla.route(q, k, 3, 4)
    np.testing.assert_array_equal(r["crit_idx"], p["crit_idx"])
    np.testing.assert_array_equal(r["marg_idx"], p["marg_idx"])
    # zero values: every M_j = 0 and the logits are the plain ones
    r0 = pisa.route_pisa(q, k, np.zeros_like(v), 3, 4)
    np.testing.assert_array_equal(r0["block_dev"], 0.0)
    np.testing.assert_array_equal(r0["logits"], p["logits"])


def test_logit_grows_with_the_block_deviation_alone():
    nq, nkb, d = 4, 10, 8
    qp, kp = rng.standard_normal((nq, d)), rng.standard_normal((nkb, d))
    M = rng.uniform(10, 60, nkb)
    base = pisa.covariance_logits(qp, kp, M)
    M2 = M.copy()
    M2[6] *= 1.5
    up = pisa.covariance_logits(qp, kp, M2)
    assert (up[:, 6] > base[:, 6]).all()
    np.testing.assert_array_equal(np.delete(up, 6, axis=1), np.delete(base, 6, axis=1))
    # raised far enough, a block enters every row's critical set
    M2[6] = 1e9
    crit, _, _ = sla.select(pisa.covariance_logits(qp, kp, M2), 2, 3)
    assert all(6 in row for row in crit)


def test_covariance_routing_lowers_the_piecewise_error_on_heterogeneous_blocks():
    # four blocks whose values follow their (spread-out) keys carry large
    # first-order matrices that the shared Hbar misses; the covariance-aware
    # split computes them exactly and the piecewise output lands closer to
    # dense attention than with the plain split
    r_ = np.random.default_rng(0)
    nb, d = 16, 16
    n = 64 * nb
    cen = r_.standard_normal((nb, d))
    k = np.repeat(cen, 64, axis=0) + 0.5 * r_.standard_normal((n, d))
    q = np.repeat(cen[r_.permutation(nb)], 64, axis=0) * 0.8 + 0.5 * r_.standard_normal((n, d))
    v = r_.standard_normal((n, d))
    W = r_.standard_normal((d, d))
    for j in r_.choice(nb, 4, replace=False):
        a, b = 64 * j, 64 * j + 64
        k[a:b] += 2.0 * r_.standard_normal((64, d))
        v[a:b] = (k[a:b] - k[a:b].mean(axis=0)) @ W * 0.5
    ref = _dense(q, k, v)
    plain = sla.route(q, k, 3, 0)["crit_idx"]
    cov = pisa.route_pisa(q, k, v, 3, 0)["crit_idx"]
    e_plain = np.linalg.norm(pisa.pisa_head(q, k, v, plain)[0] - ref) / np.linalg.norm(ref)
    e_cov = np.linalg.norm(pisa.pisa_head(q, k, v, cov)[0] - ref) / np.linalg.norm(ref)
    assert e_cov < 0.6 * e_plain, (e_cov, e_plain)
