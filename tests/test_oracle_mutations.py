"""The oracle's pins have teeth: plant a plausible mistake in the oracle and
check that the pin meant to catch it fails (CPU only)."""
import math

import numpy as np
import pytest

from oracle import sla
import tests.test_oracle_pins as pins


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_pool_dividing_by_full_block(monkeypatch):
    def bad(x, block=64):
        n, d = x.shape
        out = np.empty((sla.n_blocks(n, block), d))
        for j, (a, b) in enumerate(sla.block_ranges(n, block)):
            out[j] = x[a:b].sum(0) / block
        return out
    monkeypatch.setattr(sla, "pool", bad)
    _fails(pins.test_pool_tail_divides_by_valid_count)


def test_logits_without_scale(monkeypatch):
    monkeypatch.setattr(sla, "block_logits", lambda qp, kp: qp @ kp.T)
    _fails(pins.test_logits_brute_force)


def test_ties_to_higher_index(monkeypatch):
    orig = sla.select

    def bad(logits, kc, km):
        flipped = logits[:, ::-1]
        c, m, cls = orig(flipped, kc, km)
        nkb = logits.shape[1]
        return np.sort(nkb - 1 - c, 1), np.sort(nkb - 1 - m, 1), cls[:, ::-1]
    monkeypatch.setattr(sla, "select", bad)
    _fails(pins.test_select_matches_brute_force, 3, 5, True)


def test_sparse_without_scale(monkeypatch):
    def bad(q, k, v, crit_idx, block=64, q_blocks=None):
        return sla.__dict__["_orig_sparse"](q * math.sqrt(q.shape[1]), k, v, crit_idx, block, q_blocks)
    sla.__dict__["_orig_sparse"] = sla.sparse_branch
    monkeypatch.setattr(sla, "sparse_branch", bad)
    try:
        _fails(pins.test_all_critical_is_dense_attention, 200)
    finally:
        del sla.__dict__["_orig_sparse"]


def test_phi_over_tokens(monkeypatch):
    def bad(x):
        e = np.exp(x - x.max(axis=0, keepdims=True))
        return e / e.sum(axis=0, keepdims=True)
    monkeypatch.setattr(sla, "phi", bad)
    _fails(pins.test_phi_is_feature_softmax)
    _fails(pins.test_states_invariants, 150)


def test_transposed_states(monkeypatch):
    orig = sla.linear_states

    def bad(k, v, block=64):
        H, z = orig(k, v, block)
        return np.transpose(H, (0, 2, 1)).copy(), z
    monkeypatch.setattr(sla, "linear_states", bad)
    _fails(pins.test_states_invariants, 192)


def test_linear_without_denominator(monkeypatch):
    def bad(q, H, z, marg_idx, block=64, q_blocks=None):
        out = np.zeros((q.shape[0], H.shape[2]))
        fq = sla.phi(q)
        for i, (a, b) in enumerate(sla.block_ranges(q.shape[0], block)):
            if len(marg_idx[i]):
                out[a:b] = fq[a:b] @ H[marg_idx[i]].sum(0)
        return out
    monkeypatch.setattr(sla, "linear_branch", bad)
    _fails(pins.test_all_marginal_is_closed_form_linear_attention, 256)


def test_mix_swapped(monkeypatch):
    monkeypatch.setattr(sla, "mix", lambda o_s, o_l, a: (1 - a) * o_s + a * o_l)
    _fails(pins.test_mix_endpoints_and_affinity)


# ------------------------------------------------- residual linear attention

import oracle.rla as rla_mod
import tests.test_oracle_pins_rla as rla_pins


def test_rla_sum_instead_of_difference(monkeypatch):
    def bad(q, H, crit_idx, block=64, q_blocks=None):
        n, d = q.shape
        out = np.zeros((n, H.shape[2]))
        fq = np.exp(q - q.max(axis=1, keepdims=True))
        S_all = H.sum(axis=0)
        for i, (a, b) in enumerate(sla.block_ranges(n, block)):
            c = crit_idx[i]
            out[a:b] = fq[a:b] @ S_all + (fq[a:b] @ H[c].sum(axis=0) if len(c) else 0)
        return out
    monkeypatch.setattr(rla_mod, "rla_branch", bad)
    _fails(rla_pins.test_rla_branch_brute_force_over_noncritical_tokens, 40, 4, 8, 2)


def test_rla_states_transposed(monkeypatch):
    orig = rla_mod.linear_states_exp

    def bad(k, v, block=64):
        H, z = orig(k, v, block)
        return H.transpose(0, 2, 1).copy(), z
    monkeypatch.setattr(rla_mod, "linear_states_exp", bad)
    _fails(rla_pins.test_states_exp_brute_force, 10, 3, 4)


def test_rla_rms_over_rows(monkeypatch):
    monkeypatch.setattr(rla_mod, "rms_norm",
                        lambda x, eps=1e-6: x / np.sqrt((x * x).mean(axis=0, keepdims=True) + eps))
    _fails(rla_pins.test_rms_norm_closed_forms)


def test_rla_rms_without_eps(monkeypatch):
    monkeypatch.setattr(rla_mod, "rms_norm",
                        lambda x, eps=1e-6: x / np.sqrt((x * x).mean(axis=-1, keepdims=True)))
    _fails(rla_pins.test_rms_norm_closed_forms)


from oracle import taylor as taylor_mod
import tests.test_oracle_pins_taylor as taylor_pins


def test_taylor_without_half(monkeypatch):
    def bad(qp, kp, kv):
        d = qp.shape[1]
        return (qp @ kp.T) / math.sqrt(d) + np.log1p(((qp * qp) @ kv.T) / d)
    monkeypatch.setattr(taylor_mod, "taylor_logits", bad)
    _fails(taylor_pins.test_score_matches_block_mass_to_fourth_order, 1e-2)


def test_taylor_unscaled_second_order(monkeypatch):
    def bad(qp, kp, kv):
        d = qp.shape[1]
        return (qp @ kp.T) / math.sqrt(d) + np.log1p(((qp * qp) @ kv.T) / 2.0)
    monkeypatch.setattr(taylor_mod, "taylor_logits", bad)
    _fails(taylor_pins.test_score_matches_block_mass_to_fourth_order, 1e-2)


def test_taylor_sample_variance(monkeypatch):
    def bad(x, block=64):
        n, d = x.shape
        out = np.zeros((sla.n_blocks(n, block), d))
        for j, (a, b) in enumerate(sla.block_ranges(n, block)):
            if b - a > 1:
                out[j] = x[a:b].var(axis=0, ddof=1)
        return out
    monkeypatch.setattr(taylor_mod, "block_variance", bad)
    _fails(taylor_pins.test_block_variance_brute_force_with_short_tail)


def test_taylor_variance_of_queries(monkeypatch):
    # the spread term taken over the query blocks instead of the key blocks
    orig = taylor_mod.route_taylor

    def bad(q, k, kc, km, block=64):
        return orig(k, q, kc, km, block)
    monkeypatch.setattr(taylor_mod, "route_taylor", bad)
    _fails(taylor_pins.test_zero_variance_gives_the_sla_route)


from oracle import pisa as pisa_mod
import tests.test_oracle_pins_pisa as pisa_pins


def _patch_stats(monkeypatch, fn):
    orig = pisa_mod.block_statistics
    monkeypatch.setattr(pisa_mod, "block_statistics", lambda k, v, block=64: fn(*orig(k, v, block)))


def test_pisa_denominator_without_token_count(monkeypatch):
    _patch_stats(monkeypatch, lambda kb, vs, cnt, H: (kb, vs, np.ones_like(cnt), H))
    _fails(pisa_pins.test_constant_key_blocks_make_the_expansion_exact, 64 * 6, 2)


def test_pisa_value_mean_instead_of_sum(monkeypatch):
    _patch_stats(monkeypatch, lambda kb, vs, cnt, H: (kb, vs / cnt[:, None], cnt, H))
    _fails(pisa_pins.test_constant_key_blocks_make_the_expansion_exact, 64 * 6, 2)


def test_pisa_uncentred_first_order(monkeypatch):
    _patch_stats(monkeypatch, lambda kb, vs, cnt, H: (kb, vs, cnt,
                                                       H + kb[:, :, None] * vs[:, None, :]))
    _fails(pisa_pins.test_constant_key_blocks_make_the_expansion_exact, 64 * 6, 2)


def test_pisa_hbar_summed_not_averaged(monkeypatch):
    monkeypatch.setattr(pisa_mod, "global_first_order", lambda H: H.sum(axis=0))
    _fails(pisa_pins.test_equal_first_order_matrices_leave_second_order_error)


def test_pisa_correction_unscaled(monkeypatch):
    # the correction taken with q_t instead of q_t / sqrt(d)
    monkeypatch.setattr(pisa_mod, "global_first_order", lambda H: H.mean(axis=0) * math.sqrt(8))
    _fails(pisa_pins.test_equal_first_order_matrices_leave_second_order_error)


def test_pisa_correction_sign(monkeypatch):
    monkeypatch.setattr(pisa_mod, "global_first_order", lambda H: -H.mean(axis=0))
    _fails(pisa_pins.test_equal_first_order_matrices_leave_second_order_error)


def test_pisa_deviation_without_hbar(monkeypatch):
    # the norm of H_j itself instead of its deviation from Hbar
    monkeypatch.setattr(pisa_mod, "block_deviation",
                        lambda H, Hbar: np.sqrt((H * H).sum(axis=(1, 2))))
    _fails(pisa_pins.test_equal_deviations_give_the_plain_split)


def test_pisa_covariance_term_unscaled(monkeypatch):
    # |qbar| M_j without the 1 / (sqrt(d) B) factor
    monkeypatch.setattr(pisa_mod, "covariance_logits", lambda qp, kp, M, block=64:
                        qp @ kp.T / math.sqrt(qp.shape[1])
                        + np.log1p(np.linalg.norm(qp, axis=1)[:, None] * M[None, :]))
    _fails(pisa_pins.test_covariance_logits_brute_force)


def test_pisa_covariance_term_subtracted(monkeypatch):
    orig = pisa_mod.covariance_logits
    monkeypatch.setattr(pisa_mod, "covariance_logits", lambda qp, kp, M, block=64:
                        2 * (qp @ kp.T / math.sqrt(qp.shape[1])) - orig(qp, kp, M, block))
    _fails(pisa_pins.test_logit_grows_with_the_block_deviation_alone)


from oracle import backward as bwd_mod
import tests.test_oracle_pins_backward as bwd_pins


def test_backward_softmax_without_row_term(monkeypatch):
    orig = bwd_mod.sparse_branch_backward

    def bad(q, k, v, crit_idx, do_s, block=64):
        # drops the rowsum(dO_s * O_s) term: dS = P * dP
        n, d = q.shape
        dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
        for i, (a, b) in enumerate(sla.block_ranges(n, block)):
            c = crit_idx[i]
            if len(c) == 0:
                continue
            toks = np.concatenate([np.arange(*sla.block_ranges(n, block)[j]) for j in c])
            x = q[a:b] @ k[toks].T / math.sqrt(d)
            p = np.exp(x - x.max(axis=1, keepdims=True)); p /= p.sum(axis=1, keepdims=True)
            dv[toks] += p.T @ do_s[a:b]
            ds = p * (do_s[a:b] @ v[toks].T)
            dq[a:b] += ds @ k[toks] / math.sqrt(d)
            dk[toks] += ds.T @ q[a:b] / math.sqrt(d)
        return dq, dk, dv
    monkeypatch.setattr(bwd_mod, "sparse_branch_backward", bad)
    _fails(bwd_pins.test_gradients_match_finite_differences, 20, 1, 1, 0.6)


def test_backward_phi_jacobian_dropped(monkeypatch):
    monkeypatch.setattr(bwd_mod, "phi_backward", lambda f, df: df)
    _fails(bwd_pins.test_gradients_match_finite_differences, 24, 0, 2, 0.5)


def test_backward_alpha_sign(monkeypatch):
    orig = bwd_mod.backward_head

    def bad(q, k, v, crit_idx, marg_idx, alpha, do, block=64):
        dq, dk, dv, da = orig(q, k, v, crit_idx, marg_idx, alpha, do, block)
        return dq, dk, dv, -da
    monkeypatch.setattr(bwd_mod, "backward_head", bad)
    _fails(bwd_pins.test_gradients_match_finite_differences, 20, 1, 1, 0.6)
