"""Residual linear attention on the GPU against the fp64 oracle (oracle/rla.py).

The states use the exponential feature map; the residual state of each query
block is every KV block outside its critical list (routing with k_marg =
nkb - k_crit); the residual branch is RMS-normalised and gated with alpha.
"""
import numpy as np
import pytest
import torch

from oracle import rla as orla
from oracle import sla as ora
from tests.parity_utils import (MAX_ABS_BF16, REL_L2_BF16, format_per_head, max_abs, metrics_by_head,
                                rel_l2, to64)
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _s():
    import block_sparse_linear_route_amd as s
    return s


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name,heads", [("tiny", None), ("seq8k", None), ("video32k", None)])
def test_states_exp_parity(name, heads):
    s = _s()
    w = make_workload(name)
    k, v = w.k.to(DEV), w.v.to(DEV)
    Hs, zs = s.linear_states(k, v, feature_map="exp")
    torch.cuda.synchronize()
    B, H, N, d = w.shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    k64, v64 = to64(w.k), to64(w.v)
    for b, h in heads:
        H64, z64 = orla.linear_states_exp(k64[b, h], v64[b, h])
        hg = to64(Hs[b, h]).transpose(0, 2, 1)      # stored value-major: [j][c][a]
        zg = zs[b, h].cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(zg, z64, rtol=2e-5, atol=1e-6)
        err = rel_l2(hg, H64)
        _say(f"[states exp {name} b{b}h{h}] H rel L2 {err:.2e} max-abs {max_abs(hg, H64):.2e}")
        assert err < 5e-3
        assert max_abs(hg, H64) < 2e-2 * max(1.0, np.abs(H64).max())


def _rla_check(w, kc, heads=None, n_sample=None, seed=0, form="complement"):
    s = _s()
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    B, H, N, d = w.shape
    nb = ora.n_blocks(N)
    r = s.route(q, k, kc, nb - kc)
    Hs, _ = s.linear_states(k, v, feature_map="exp")
    if form == "complement":
        o, o_s, o_l = s.forward_rla(q, k, v, r["crit_idx"], Hs, w.alpha, branches=True)
    else:
        # the subtraction form: global state minus the critical blocks' states
        ws = s.residual_workspace_subtract(q, kc)
        s.residual_sums_subtract(q, r["crit_idx"], Hs, ws)
        o, o_s, o_l = s.forward_attend_rla(q, k, v, r["crit_idx"], w.alpha, ws, branches=True)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(w.q), to64(w.k), to64(w.v)
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    rng = np.random.default_rng(seed)
    pairs = {"o": {}, "s": {}, "l": {}}
    og, osg, olg = to64(o), o_s.cpu().numpy(), o_l.cpu().numpy()
    for b, h in heads:
        crit = r["crit_idx"][b, h].cpu().numpy().astype(np.int64)
        marg = r["marg_idx"][b, h].cpu().numpy().astype(np.int64)
        # the router's marginal list is exactly the complement of the critical one
        both = np.sort(np.concatenate([crit, marg], axis=1), axis=1)
        assert np.array_equal(both, np.broadcast_to(np.arange(nb), both.shape))
        if n_sample is None or n_sample >= nb:
            qb = list(range(nb))
        else:
            qb = sorted(set(rng.choice(nb - 1, n_sample - 1, replace=False).tolist()) | {nb - 1})
        He, _ = orla.linear_states_exp(k64[b, h], v64[b, h])
        ro, rs, rn = orla.forward_head_rla(q64[b, h], k64[b, h], v64[b, h], crit, He,
                                           float(w.alpha[h]), q_blocks=qb)
        rows = np.concatenate([np.arange(64 * i, min(64 * i + 64, N)) for i in qb])
        lab = f"b{b}h{h}"
        pairs["o"][lab] = (og[b, h][rows], ro[rows])
        pairs["s"][lab] = (osg[b, h][rows].astype(np.float64), rs[rows])
        pairs["l"][lab] = (olg[b, h][rows].astype(np.float64), rn[rows])
    res, per = {}, {}
    for key in ("o", "s", "l"):
        res[key], per[key] = metrics_by_head(pairs[key])
    _say(f"[rla {form} {w.name} N={N} d={d} kc={kc} {w.q.dtype}; {len(heads)} heads] "
         + " ".join(f"{k_}: relL2 {v_[0]:.2e} maxabs {v_[1]:.2e}" for k_, v_ in res.items()))
    if len(heads) > 1:
        _say("  per head O relL2/maxabs: " + format_per_head(per["o"]))
    for key in ("o", "s", "l"):
        if key == "s" and kc == 0 or key == "l" and kc == nb:
            assert res[key][1] == 0.0
            continue
        assert res[key][0] <= REL_L2_BF16, (key, res[key])
        assert res[key][1] <= MAX_ABS_BF16, (key, res[key])
    for lab, (e, m) in per["o"].items():
        assert e <= REL_L2_BF16 and m <= MAX_ABS_BF16, (lab, e, m)
    return res


@pytest.mark.parametrize("name,heads,n_sample", [
    ("tiny", None, None), ("seq8k", None, None),
    pytest.param("video32k", None, None, marks=pytest.mark.timeout(900))])
def test_forward_rla_parity(name, heads, n_sample):
    w = make_workload(name)
    _rla_check(w, w.k_crit, heads, n_sample)


@pytest.mark.parametrize("N,d,dtype,kc,H,seed", [
    (1000, 128, "bf16", 0, 2, 60),        # nothing critical: everything residual
    (1000, 128, "bf16", 16, 1, 61),       # everything critical: empty residual state
    (777, 64, "fp32", 3, 2, 62),
    (4095, 128, "bf16", 1, 1, 63),
    (65, 128, "bf16", 1, 1, 64),          # two blocks, the second one row long
    # critical lists past the 64 entries one list register holds
    (300 * 64 + 17, 128, "bf16", 65, 1, 66),
    (300 * 64 + 17, 128, "bf16", 129, 1, 67),
    (270 * 64, 128, "bf16", 260, 1, 68),
])
def test_forward_rla_parity_shapes(N, d, dtype, kc, H, seed):
    nb = ora.n_blocks(N)
    w = make_custom(1, H, N, d, dtype=dtype, kind="fourier1d", seed=seed, k_crit=kc,
                    k_marg=nb - kc)
    _rla_check(w, kc, n_sample=None if nb <= 64 else 48)


@pytest.mark.parametrize("name", ["tiny", "seq8k", pytest.param("video32k", marks=pytest.mark.timeout(900))])
def test_forward_rla_subtraction_form_parity(name):
    # SPLA summary, section 2.2: o_rla = o_bar - o_tilde with o_bar from the
    # head's global state and o_tilde from the selected blocks only
    w = make_workload(name)
    _rla_check(w, w.k_crit, form="subtract")


@pytest.mark.parametrize("N,d,dtype,kc,H,seed", [
    (1000, 128, "bf16", 0, 2, 60),        # nothing selected: the global state alone
    (1000, 128, "bf16", 15, 1, 61),       # one residual block left
    (777, 64, "fp32", 3, 2, 62),
    (300 * 64 + 17, 128, "bf16", 129, 1, 67),
])
def test_forward_rla_subtraction_form_shapes(N, d, dtype, kc, H, seed):
    nb = ora.n_blocks(N)
    w = make_custom(1, H, N, d, dtype=dtype, kind="fourier1d", seed=seed, k_crit=kc,
                    k_marg=nb - kc)
    _rla_check(w, kc, n_sample=None if nb <= 64 else 48, form="subtract")


def test_forward_rla_phases_equal_fused_call():
    s = _s()
    w = make_custom(1, 2, 3000, 128, seed=65, k_crit=5, k_marg=ora.n_blocks(3000) - 5)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    nb = ora.n_blocks(3000)
    r = s.route(q, k, 5, nb - 5)
    Hs, _ = s.linear_states(k, v, feature_map="exp")
    o1 = s.forward_rla(q, k, v, r["crit_idx"], Hs, w.alpha)
    ws = s.forward_workspace(q, 5, nb - 5)
    s.residual_sums(q, r["crit_idx"], Hs, ws)
    o2 = s.forward_attend_rla(q, k, v, r["crit_idx"], w.alpha, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.timeout(900)
def test_forward_rla_parity_video75k():
    # every head, 32 sampled query blocks each (the last one included)
    w = make_workload("video75k")
    _rla_check(w, w.k_crit, n_sample=32)
