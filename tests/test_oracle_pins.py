"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one oracle step to a closed form, an invariant, a special
case that reduces to a library routine, or brute force on tiny inputs, so a
dropped term, a wrong sign or index or a transposed operand in the oracle
fails at least one of them.  ``test_oracle_mutations.py`` plants such
mistakes and checks that these pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import sla

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(7)


# ----------------------------------------------------------------- pooling

@pytest.mark.parametrize("n,block", [(248, 64), (1000, 64), (75600 % 640 + 64 * 3, 64), (10, 4)])
def test_pool_constant_blocks_pool_to_themselves(n, block):
    d = 6
    nb = sla.n_blocks(n, block)
    vals = rng.integers(-40, 40, size=(nb, d)) / 8.0     # dyadic: sums are exact
    x = np.repeat(vals, block, axis=0)[:n]
    np.testing.assert_array_equal(sla.pool(x, block), vals)


def test_pool_tail_divides_by_valid_count():
    x = np.ones((64 * 2 + 56, 3))
    x[128:] = 5.0
    p = sla.pool(x, 64)
    assert p.shape == (3, 3)
    np.testing.assert_array_equal(p[2], [5.0, 5.0, 5.0])


def test_pool_is_linear():
    x = rng.standard_normal((200, 8))
    y = rng.standard_normal((200, 8))
    np.testing.assert_allclose(sla.pool(2.5 * x - 0.5 * y), 2.5 * sla.pool(x) - 0.5 * sla.pool(y),
                               rtol=1e-13, atol=1e-13)


def test_pool_brute_force():
    n, d, blk = 11, 3, 4
    x = rng.standard_normal((n, d))
    out = sla.pool(x, blk)
    for j in range(3):
        rows = [r for r in range(n) if r // blk == j]
        for c in range(d):
            acc = 0.0
            for r in rows:
                acc += x[r, c]
            assert math.isclose(out[j, c], acc / len(rows), rel_tol=1e-14, abs_tol=1e-15)


# ----------------------------------------------------------------- routing

def test_logits_brute_force():
    qp = rng.standard_normal((5, 7))
    kp = rng.standard_normal((6, 7))
    s = sla.block_logits(qp, kp)
    for i in range(5):
        for j in range(6):
            acc = sum(qp[i, a] * kp[j, a] for a in range(7))
            assert math.isclose(s[i, j], acc / math.sqrt(7), rel_tol=1e-13, abs_tol=1e-14)


def _brute_select(s, kc, km):
    nq, nkb = s.shape
    crit, marg, cls = [], [], np.zeros((nq, nkb), dtype=np.int8)
    for i in range(nq):
        order = sorted(range(nkb), key=lambda j: (-s[i, j], j))
        c = sorted(order[:kc])
        m = sorted(order[kc:kc + km])
        crit.append(c)
        marg.append(m)
        for j in c:
            cls[i, j] = 2
        for j in m:
            cls[i, j] = 1
    return np.array(crit, dtype=np.int64).reshape(nq, kc), np.array(marg, dtype=np.int64).reshape(nq, km), cls


@pytest.mark.parametrize("kc,km", [(3, 5), (0, 4), (4, 0), (6, 10), (1, 15), (16, 0), (0, 16)])
@pytest.mark.parametrize("ties", [False, True])
def test_select_matches_brute_force(kc, km, ties):
    s = rng.standard_normal((9, 16))
    if ties:
        s = np.round(s, 1)      # many equal logits: the lower block index must win
        s[0, :] = 0.0
        s[1, ::2] = -0.0        # -0.0 and 0.0 are the same logit
    crit, marg, cls = sla.select(s, kc, km)
    bc, bm, bcls = _brute_select(s, kc, km)
    np.testing.assert_array_equal(crit, bc)
    np.testing.assert_array_equal(marg, bm)
    np.testing.assert_array_equal(cls, bcls)


def test_select_class_counts_disjoint_cover():
    s = rng.standard_normal((40, 33))
    crit, marg, cls = sla.select(s, 5, 9)
    assert ((cls == 2).sum(1) == 5).all() and ((cls == 1).sum(1) == 9).all()
    assert ((cls == 0).sum(1) == 33 - 14).all()
    for i in range(40):
        assert len(set(crit[i]) & set(marg[i])) == 0
        assert (np.diff(crit[i]) > 0).all() and (np.diff(marg[i]) > 0).all()
        # every critical logit is >= every marginal logit >= every negligible one
        neg = np.nonzero(cls[i] == 0)[0]
        assert s[i, crit[i]].min() >= s[i, marg[i]].max() >= s[i, neg].max()


def test_ranking_on_logits_equals_ranking_on_block_softmax():
    # the block-score map is softmax over j; ranking on it equals ranking on s
    s = rng.standard_normal((12, 40)) * 3
    p = scipy.special.softmax(s, axis=1)
    a = np.argsort(-s, axis=1, kind="stable")
    b = np.argsort(-p, axis=1, kind="stable")
    np.testing.assert_array_equal(a, b)
    crit, marg, _ = sla.select(s, 4, 8)
    crit_p, marg_p, _ = sla.select(p, 4, 8)
    np.testing.assert_array_equal(crit, crit_p)
    np.testing.assert_array_equal(marg, marg_p)


def test_select_rejects_bad_counts():
    with pytest.raises(ValueError):
        sla.select(np.zeros((2, 4)), 3, 2)


# ----------------------------------------------------------------- sparse branch

def _dense_attention(q, k, v):
    s = q @ k.T / math.sqrt(q.shape[1])
    return scipy.special.softmax(s, axis=1) @ v


@pytest.mark.parametrize("n", [200, 256, 130])
def test_all_critical_is_dense_attention(n):
    d = 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    nkb = sla.n_blocks(n)
    r = sla.route(q, k, nkb, 0)
    o_s = sla.sparse_branch(q, k, v, r["crit_idx"])
    np.testing.assert_allclose(o_s, _dense_attention(q, k, v), rtol=1e-12, atol=1e-12)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    np.testing.assert_allclose(o_s, ref, rtol=1e-10, atol=1e-12)
    # and through the full mix at alpha = 1 (the linear branch is empty)
    H, z = sla.linear_states(k, v)
    o, _, o_l = sla.forward_head(q, k, v, r["crit_idx"], r["marg_idx"], H, z, 1.0)
    np.testing.assert_array_equal(o_l, 0.0)
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def test_zero_query_gives_mean_of_critical_values():
    n, d = 192 + 20, 8
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    q = np.zeros((n, d))
    crit = np.array([[0, 3], [1, 2], [2, 3], [0, 1]])
    o_s = sla.sparse_branch(q, k, v, crit)
    for i in range(4):
        toks = [t for j in crit[i] for t in range(j * 64, min(j * 64 + 64, n))]
        mean = v[toks].mean(axis=0)
        for t in range(i * 64, min(i * 64 + 64, n)):
            np.testing.assert_allclose(o_s[t], mean, rtol=1e-12, atol=1e-13)


def test_sparse_branch_per_token_brute_force():
    n, d, blk = 9, 3, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    crit = np.array([[0, 2], [1, 2], [0, 1]])
    o_s = sla.sparse_branch(q, k, v, crit, blk)
    for t in range(n):
        i = t // blk
        keys = [u for j in crit[i] for u in range(j * blk, min(j * blk + blk, n))]
        w = [math.exp(sum(q[t, a] * k[u, a] for a in range(d)) / math.sqrt(d)) for u in keys]
        for c in range(d):
            num = sum(wi * v[u, c] for wi, u in zip(w, keys))
            assert math.isclose(o_s[t, c], num / sum(w), rel_tol=1e-11, abs_tol=1e-12)


def test_empty_critical_set_gives_zero():
    n, d = 128, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o_s = sla.sparse_branch(q, k, v, np.zeros((2, 0), dtype=np.int64))
    np.testing.assert_array_equal(o_s, 0.0)


# ----------------------------------------------------------------- states

def test_phi_is_feature_softmax():
    x = rng.standard_normal((7, 11)) * 4
    np.testing.assert_allclose(sla.phi(x), scipy.special.softmax(x, axis=1), rtol=1e-14)


@pytest.mark.parametrize("n", [192, 150])
def test_states_invariants(n):
    d = 12
    k, v = rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d))
    H, z = sla.linear_states(k, v)
    for j, (a, b) in enumerate(sla.block_ranges(n)):
        assert math.isclose(z[j].sum(), b - a, rel_tol=1e-13)
        np.testing.assert_allclose(H[j].sum(axis=0), v[a:b].sum(axis=0), rtol=1e-12, atol=1e-12)


def test_states_constant_key_rows():
    n, d = 150, 10
    k = np.repeat(rng.standard_normal((n, 1)), d, axis=1)   # equal features per row
    v = rng.standard_normal((n, d))
    H, z = sla.linear_states(k, v)
    for j, (a, b) in enumerate(sla.block_ranges(n)):
        np.testing.assert_allclose(H[j], np.outer(np.ones(d), v[a:b].sum(0)) / d, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(z[j], np.full(d, (b - a) / d), rtol=1e-14)


def test_states_brute_force():
    n, d, blk = 6, 3, 4
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    H, z = sla.linear_states(k, v, blk)
    for j, (a, b) in enumerate(sla.block_ranges(n, blk)):
        for t in range(a, b):
            pass
        for x in range(d):
            zz = 0.0
            for t in range(a, b):
                e = [math.exp(k[t, c]) for c in range(d)]
                zz += e[x] / sum(e)
            assert math.isclose(z[j, x], zz, rel_tol=1e-13)
            for y in range(d):
                hh = 0.0
                for t in range(a, b):
                    e = [math.exp(k[t, c]) for c in range(d)]
                    hh += e[x] / sum(e) * v[t, y]
                assert math.isclose(H[j, x, y], hh, rel_tol=1e-12, abs_tol=1e-14)


# ----------------------------------------------------------------- linear branch

@pytest.mark.parametrize("n", [256, 200])
def test_all_marginal_is_closed_form_linear_attention(n):
    d = 16
    q, k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    nkb = sla.n_blocks(n)
    r = sla.route(q, k, 0, nkb)
    H, z = sla.linear_states(k, v)
    o_l = sla.linear_branch(q, H, z, r["marg_idx"])
    # quadratic form, no states: A = phi(Q) phi(K)^T, O = A V / (A 1)
    A = scipy.special.softmax(q, axis=1) @ scipy.special.softmax(k, axis=1).T
    np.testing.assert_allclose(o_l, (A @ v) / A.sum(1, keepdims=True), rtol=1e-11, atol=1e-12)
    o, o_s, _ = sla.forward_head(q, k, v, r["crit_idx"], r["marg_idx"], H, z, 0.0)
    np.testing.assert_array_equal(o_s, 0.0)
    np.testing.assert_allclose(o, (A @ v) / A.sum(1, keepdims=True), rtol=1e-11, atol=1e-12)


def test_uniform_phi_query_gives_mean_of_marginal_values():
    n, d = 256, 8
    q = np.repeat(rng.standard_normal((n, 1)), d, axis=1)
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    marg = np.array([[1, 2], [0, 3], [0, 1], [2, 3]])
    H, z = sla.linear_states(k, v)
    o_l = sla.linear_branch(q, H, z, marg)
    for i in range(4):
        toks = [t for j in marg[i] for t in range(j * 64, j * 64 + 64)]
        np.testing.assert_allclose(o_l[i * 64:(i + 1) * 64], np.broadcast_to(v[toks].mean(0), (64, d)),
                                   rtol=1e-12, atol=1e-13)


def test_unnormalised_exp_feature_map_for_queries_gives_same_output():
    # the row normaliser of phi(q) cancels between numerator and denominator
    n, d = 192, 16
    q, k, v = rng.standard_normal((n, d)) * 3, rng.standard_normal((n, d)), rng.standard_normal((n, d))
    marg = np.array([[0, 2], [1, 2], [0, 1]])
    H, z = sla.linear_states(k, v)
    o_l = sla.linear_branch(q, H, z, marg)
    e = np.exp(q - q.max(1, keepdims=True))
    for i in range(3):
        S, sig = H[marg[i]].sum(0), z[marg[i]].sum(0)
        blk = e[i * 64:(i + 1) * 64]
        np.testing.assert_allclose(o_l[i * 64:(i + 1) * 64], (blk @ S) / (blk @ sig)[:, None],
                                   rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- mix

def test_mix_endpoints_and_affinity():
    n, d = 256, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    r = sla.route(q, k, 1, 2)
    H, z = sla.linear_states(k, v)
    o0, o_s, o_l = sla.forward_head(q, k, v, r["crit_idx"], r["marg_idx"], H, z, 0.0)
    o1, _, _ = sla.forward_head(q, k, v, r["crit_idx"], r["marg_idx"], H, z, 1.0)
    oa, _, _ = sla.forward_head(q, k, v, r["crit_idx"], r["marg_idx"], H, z, 0.3)
    np.testing.assert_array_equal(o1, o_s)
    np.testing.assert_array_equal(o0, o_l)
    np.testing.assert_allclose(oa, o0 + 0.3 * (o1 - o0), rtol=1e-12, atol=1e-13)
    assert not np.allclose(o_s, o_l)


# ----------------------------------------------------------------- worked example

def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    q, k, v = (np.array(g[x], dtype=np.float64) for x in ("q", "k", "v"))
    blk = g["block"]
    r = sla.attention_head(q, k, v, g["alpha"], g["k_crit"], g["k_marg"], blk)
    np.testing.assert_array_equal(r["crit_idx"], g["expected_crit_idx"])
    np.testing.assert_array_equal(r["marg_idx"], g["expected_marg_idx"])
    np.testing.assert_array_equal(r["block_class"], g["expected_block_class"])
    np.testing.assert_allclose(r["z"], g["expected_z"], rtol=1e-15)
    np.testing.assert_allclose(r["H"].sum(axis=1), g["expected_column_sums_of_H"], rtol=1e-15)
    # closed forms from the derivation in the fixture
    e = math.exp(math.sqrt(2.0))
    v0, v1, v2, v3 = v
    os_hot = (e * v0 + v1) / (e + 1)
    os_zero = (v0 + v1) / 2
    o_l = (v2 + v3) / 2
    np.testing.assert_allclose(r["o_sparse"], [os_hot, os_zero, os_hot, os_zero], rtol=1e-14)
    np.testing.assert_allclose(r["o_linear"], [o_l] * 4, rtol=1e-14)
    a = g["alpha"]
    np.testing.assert_allclose(r["o"], [a * x + (1 - a) * o_l for x in (os_hot, os_zero, os_hot, os_zero)],
                               rtol=1e-14)


# ----------------------------------------------------------------- end-to-end brute force

def test_pipeline_brute_force_tiny():
    n, d, blk, kc, km = 10, 3, 4, 1, 1
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    r = sla.attention_head(q, k, v, 0.7, kc, km, blk)
    nb = 3
    rows = [[t for t in range(n) if t // blk == j] for j in range(nb)]
    mean = lambda x, rr: [sum(x[t, c] for t in rr) / len(rr) for c in range(d)]
    qb = [mean(q, rows[j]) for j in range(nb)]
    kb = [mean(k, rows[j]) for j in range(nb)]

    def phi_row(x):
        e = [math.exp(x[c]) for c in range(d)]
        return [ei / sum(e) for ei in e]

    for i in range(nb):
        s = [sum(qb[i][c] * kb[j][c] for c in range(d)) / math.sqrt(d) for j in range(nb)]
        order = sorted(range(nb), key=lambda j: (-s[j], j))
        C, M = order[:kc], order[kc:kc + km]
        assert list(r["crit_idx"][i]) == sorted(C) and list(r["marg_idx"][i]) == sorted(M)
        keys = [u for j in sorted(C) for u in rows[j]]
        mtoks = [u for j in sorted(M) for u in rows[j]]
        for t in rows[i]:
            w = [math.exp(sum(q[t, c] * k[u, c] for c in range(d)) / math.sqrt(d)) for u in keys]
            pq = phi_row(q[t])
            wl = [sum(pq[c] * phi_row(k[u])[c] for c in range(d)) for u in mtoks]
            for c in range(d):
                o_s = sum(wi * v[u, c] for wi, u in zip(w, keys)) / sum(w)
                o_l = sum(wi * v[u, c] for wi, u in zip(wl, mtoks)) / sum(wl)
                assert math.isclose(r["o"][t, c], 0.7 * o_s + 0.3 * o_l, rel_tol=1e-11, abs_tol=1e-12)
