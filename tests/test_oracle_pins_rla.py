"""Pins of the residual-linear-attention oracle (oracle/rla.py), CPU only.

Each test ties one step to brute force over tokens, a closed form or a
special case of the SLA oracle, so a flipped sign in o_bar - o_tilde, a
missing block, a transposed state or a wrong RMS-norm axis fails one of them.
"""
import math

import numpy as np
import pytest

from oracle import rla, sla

rng = np.random.default_rng(11)


def _qkv(n, d, dv=None, scale=0.5):
    dv = dv or d
    return (rng.standard_normal((n, d)) * scale, rng.standard_normal((n, d)) * scale,
            rng.standard_normal((n, dv)))


@pytest.mark.parametrize("n,d,block", [(10, 3, 4), (17, 5, 8), (64, 4, 64)])
def test_states_exp_brute_force(n, d, block):
    _, k, v = _qkv(n, d, d + 1)
    H, z = rla.linear_states_exp(k, v, block)
    for j, (a, b) in enumerate(sla.block_ranges(n, block)):
        for r in range(d):
            zz = 0.0
            for t in range(a, b):
                zz += math.exp(k[t, r])
            assert abs(z[j, r] - zz) <= 1e-12 * abs(zz)
            for c in range(d + 1):
                acc = 0.0
                for t in range(a, b):
                    acc += math.exp(k[t, r]) * v[t, c]
                assert abs(H[j, r, c] - acc) <= 1e-12 * (1 + abs(acc))


def test_states_exp_is_scaled_softmax_state_for_equal_row_sums():
    # keys that are permutations of one vector share sum_a exp(k_a) = s, so
    # exp(k) = s * softmax(k) token by token and H_exp = s * H_softmax
    d, n, block = 6, 24, 8
    base = rng.standard_normal(d)
    k = np.stack([rng.permutation(base) for _ in range(n)])
    v = rng.standard_normal((n, d))
    s = np.exp(base).sum()
    He, ze = rla.linear_states_exp(k, v, block)
    Hs, zs = sla.linear_states(k, v, block)
    np.testing.assert_allclose(He, s * Hs, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ze, s * zs, rtol=1e-12)


@pytest.mark.parametrize("n,d,block,kc", [(40, 4, 8, 2), (37, 3, 8, 0), (33, 5, 16, 3)])
def test_rla_branch_brute_force_over_noncritical_tokens(n, d, block, kc):
    q, k, v = _qkv(n, d)
    nb = sla.n_blocks(n, block)
    crit = np.stack([np.sort(rng.choice(nb, kc, replace=False)) for _ in range(nb)]) if kc \
        else np.zeros((nb, 0), dtype=np.int64)
    H, _ = rla.linear_states_exp(k, v, block)
    got = rla.rla_branch(q, H, crit, block)
    ranges = sla.block_ranges(n, block)
    for i, (a, b) in enumerate(ranges):
        crit_tok = set()
        for j in crit[i]:
            crit_tok.update(range(*ranges[j]))
        for t in range(a, b):
            m = max(q[t])
            want = np.zeros(d)
            for nn in range(n):
                if nn in crit_tok:
                    continue
                w = sum(math.exp(q[t, r] - m) * math.exp(k[nn, r]) for r in range(d))
                want += w * v[nn]
            np.testing.assert_allclose(got[t], want, rtol=1e-11, atol=1e-11)


def test_rla_with_every_block_critical_is_zero():
    n, d, block = 48, 4, 8
    q, k, v = _qkv(n, d)
    nb = sla.n_blocks(n, block)
    crit = np.tile(np.arange(nb), (nb, 1))
    H, _ = rla.linear_states_exp(k, v, block)
    assert np.abs(rla.rla_branch(q, H, crit, block)).max() < 1e-12 * np.abs(H).max() * d


def test_rms_norm_closed_forms():
    x = rng.standard_normal((7, 12)) * rng.uniform(0.1, 10.0, (7, 1))
    m = (x * x).mean(axis=1)
    y = rla.rms_norm(x)
    np.testing.assert_allclose((y * y).mean(axis=1), m / (m + rla.RMS_EPS), rtol=1e-12)
    # a row of mean square 1 - eps comes out unchanged
    u = rng.standard_normal(12)
    u *= math.sqrt((1 - rla.RMS_EPS) / (u * u).mean())
    np.testing.assert_allclose(rla.rms_norm(u[None])[0], u, rtol=1e-12)
    # the norm is per row: scaling one row leaves the others alone
    x2 = x.copy()
    x2[3] *= 1e3
    np.testing.assert_allclose(rla.rms_norm(x2)[[0, 1, 2, 4, 5, 6]],
                               y[[0, 1, 2, 4, 5, 6]], rtol=1e-12)


@pytest.mark.parametrize("alpha", [0.0, 1.0, 0.35])
def test_forward_rla_mix_and_endpoints(alpha):
    n, d, block = 70, 8, 16
    q, k, v = _qkv(n, d)
    nb = sla.n_blocks(n, block)
    crit = np.stack([np.sort(rng.choice(nb, 2, replace=False)) for _ in range(nb)])
    H, _ = rla.linear_states_exp(k, v, block)
    o, o_s, o_n = rla.forward_head_rla(q, k, v, crit, H, alpha, block)
    np.testing.assert_allclose(o_s, sla.sparse_branch(q, k, v, crit, block), rtol=1e-13)
    np.testing.assert_allclose(o_n, rla.rms_norm(rla.rla_branch(q, H, crit, block)), rtol=1e-13)
    np.testing.assert_allclose(o, alpha * o_s + (1 - alpha) * o_n, rtol=1e-13, atol=1e-15)


def test_rla_output_independent_of_query_row_scale():
    # the RMS norm removes the per-row factor exp(-max q) of phi(q): with
    # phi(q) = exp(q) the normalised output agrees to far below the tolerance
    n, d, block = 64, 8, 16
    q, k, v = _qkv(n, d)
    nb = sla.n_blocks(n, block)
    crit = np.stack([np.array([i]) for i in range(nb)])
    H, _ = rla.linear_states_exp(k, v, block)
    got = rla.rms_norm(rla.rla_branch(q, H, crit, block))
    S_all = H.sum(axis=0)
    raw = np.empty((n, d))
    for i, (a, b) in enumerate(sla.block_ranges(n, block)):
        raw[a:b] = np.exp(q[a:b]) @ (S_all - H[i])
    # the two differ only through eps: per row by a factor within eps / (mean square)
    o_r = rla.rla_branch(q, H, crit, block)
    ms = np.minimum((o_r * o_r).mean(axis=1), (raw * raw).mean(axis=1))
    bound = 2 * rla.RMS_EPS / ms
    rel = np.abs(got - rla.rms_norm(raw)).max(axis=1) / np.abs(got).max(axis=1)
    assert np.all(rel <= bound + 1e-13), (rel.max(), bound.min())


def test_forward_rla_q_blocks_subset_matches_full():
    n, d, block = 90, 4, 16
    q, k, v = _qkv(n, d)
    nb = sla.n_blocks(n, block)
    crit = np.stack([np.sort(rng.choice(nb, 2, replace=False)) for _ in range(nb)])
    H, _ = rla.linear_states_exp(k, v, block)
    full = rla.forward_head_rla(q, k, v, crit, H, 0.4, block)
    part = rla.forward_head_rla(q, k, v, crit, H, 0.4, block, q_blocks=[1, 5])
    for i in (1, 5):
        a, b = sla.block_ranges(n, block)[i]
        for x, y in zip(full, part):
            np.testing.assert_allclose(y[a:b], x[a:b], rtol=1e-13)
    a, b = sla.block_ranges(n, block)[0]
    assert np.all(part[0][a:b] == 0)
