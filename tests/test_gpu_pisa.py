"""Piecewise exact-or-approximate attention on the GPU against the fp64 oracle (oracle/pisa.py).

The selected set of each query block is the router's critical list (the GPU
router's own lists, so parity does not depend on tie resolution); every
other KV block enters through its centroid, plus the global first-order
correction.  The output and its two parts (softmax part, correction part)
are held to the bf16 bar: relative L2 <= 1e-2 and max-abs <= 2e-2.
"""
import numpy as np
import pytest
import torch

from oracle import pisa as opisa
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


def _pisa_check(w, kc, heads=None, n_sample=None, seed=0):
    s = _s()
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    B, H, N, d = w.shape
    nb = ora.n_blocks(N)
    r = s.route(q, k, kc, nb - kc)
    o, o_sm, o_fo = s.forward_pisa(q, k, v, r["crit_idx"], branches=True)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(w.q), to64(w.k), to64(w.v)
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    rng = np.random.default_rng(seed)
    pairs = {"o": {}, "s": {}, "c": {}}
    og, osg, ocg = to64(o), o_sm.cpu().numpy(), o_fo.cpu().numpy()
    for b, h in heads:
        crit = r["crit_idx"][b, h].cpu().numpy().astype(np.int64)
        if n_sample is None or n_sample >= nb:
            qb = list(range(nb))
        else:
            qb = sorted(set(rng.choice(nb - 1, n_sample - 1, replace=False).tolist()) | {nb - 1})
        ro, rs, rc = opisa.pisa_head(q64[b, h], k64[b, h], v64[b, h], crit, q_blocks=qb)
        rows = np.concatenate([np.arange(64 * i, min(64 * i + 64, N)) for i in qb])
        lab = f"b{b}h{h}"
        for key, g_, r_ in (("o", og, ro), ("s", osg, rs), ("c", ocg, rc)):
            pairs[key][lab] = (g_[b, h][rows].astype(np.float64), r_[rows])
    res, per = {}, {}
    for key in ("o", "s", "c"):
        res[key], per[key] = metrics_by_head(pairs[key])
        ref_all = np.concatenate([bb.ravel() for _, bb in pairs[key].values()])
        res[key] = res[key] + (float(np.sqrt((ref_all ** 2).mean())),)
    _say(f"[pisa {w.name} N={N} d={d} kc={kc} {w.q.dtype}; {len(heads)} heads] "
         + " ".join(f"{k_}: relL2 {v_[0]:.2e} maxabs {v_[1]:.2e} (rms {v_[2]:.2e})"
                    for k_, v_ in res.items()))
    if len(heads) > 1:
        _say("  per head O relL2/maxabs: " + format_per_head(per["o"]))
    for key in ("o", "s", "c"):
        if key == "c" and kc == nb:
            assert res[key][1] == 0.0        # nothing approximated: no correction
            continue
        assert res[key][0] <= REL_L2_BF16, (key, res[key])
        assert res[key][1] <= MAX_ABS_BF16, (key, res[key])
    for lab, (e, m) in per["o"].items():
        assert e <= REL_L2_BF16 and m <= MAX_ABS_BF16, (lab, e, m)
    return res


@pytest.mark.parametrize("name,heads,n_sample", [
    ("tiny", None, None), ("seq8k", None, None),
    pytest.param("video32k", None, None, marks=pytest.mark.timeout(900))])
def test_forward_pisa_parity(name, heads, n_sample):
    w = make_workload(name)
    _pisa_check(w, w.k_crit, heads, n_sample)


@pytest.mark.parametrize("N,d,dtype,kc,H,seed", [
    (1000, 128, "bf16", 0, 2, 80),        # nothing exact: every block by its centroid
    (1000, 128, "bf16", 16, 1, 81),       # everything exact: dense attention
    (777, 64, "fp32", 3, 2, 82),
    (4095, 128, "bf16", 2, 1, 83),
    (65, 128, "bf16", 1, 1, 84),          # two blocks, the second one row long
    (64 * 70 + 5, 128, "bf16", 7, 1, 85), # two pseudo-blocks of centroids, ragged
    # critical lists past the 64 entries one list register holds, followed
    # by the centroid pseudo-blocks
    (300 * 64 + 17, 128, "bf16", 64, 1, 88),
    (300 * 64 + 17, 128, "bf16", 65, 1, 89),
    (300 * 64 + 17, 128, "bf16", 129, 1, 90),
    (270 * 64, 64, "bf16", 260, 1, 91),
])
def test_forward_pisa_parity_shapes(N, d, dtype, kc, H, seed):
    w = make_custom(1, H, N, d, dtype=dtype, kind="fourier1d", seed=seed, k_crit=kc, k_marg=0)
    _pisa_check(w, kc, n_sample=None if ora.n_blocks(N) <= 64 else 48)


@pytest.mark.parametrize("name,N", [("tiny", None), ("custom", 64 * 70 + 5)])
def test_pisa_hbar_parity(name, N):
    s = _s()
    w = make_workload("tiny") if name == "tiny" else make_custom(1, 2, N, 128, seed=86, k_crit=3,
                                                                 k_marg=0)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    ws = s.pisa_workspace(q)
    hb = s.pisa_statistics(k, v, ws, want_hbar=True)
    torch.cuda.synchronize()
    k64, v64 = to64(w.k), to64(w.v)
    B, H = w.shape[:2]
    for b in range(B):
        for h in range(H):
            _, _, _, Hj = opisa.block_statistics(k64[b, h], v64[b, h])
            ref = opisa.global_first_order(Hj)
            got = hb[b, h].cpu().numpy().astype(np.float64).T     # stored value-major
            err = rel_l2(got, ref)
            _say(f"[pisa Hbar {w.name} b{b}h{h}] rel L2 {err:.2e}")
            assert err < 5e-3


def test_forward_pisa_phases_equal_fused_call():
    s = _s()
    w = make_custom(1, 2, 3000, 128, seed=87, k_crit=5, k_marg=0)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    r = s.route(q, k, 5, 0)
    o1 = s.forward_pisa(q, k, v, r["crit_idx"])
    ws = s.pisa_workspace(q)
    s.pisa_statistics(k, v, ws)
    o2 = s.forward_attend_pisa(q, k, v, r["crit_idx"], ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_forward_pisa_beats_dropping_the_unselected_blocks():
    # on the 8k-token workload the approximate terms bring the output closer
    # to dense attention than the exact sparse branch alone
    s = _s()
    w = make_workload("seq8k")
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    r = s.route(q, k, w.k_crit, 0)
    o = s.forward_pisa(q, k, v, r["crit_idx"])
    torch.cuda.synchronize()
    q64, k64, v64 = to64(w.q)[0, 0], to64(w.k)[0, 0], to64(w.v)[0, 0]
    crit = r["crit_idx"][0, 0].cpu().numpy().astype(np.int64)
    qb = list(range(0, 128, 8))
    rows = np.concatenate([np.arange(64 * i, 64 * i + 64) for i in qb])
    dense = np.zeros_like(q64)
    x = q64[rows] @ k64.T / np.sqrt(128)
    x = np.exp(x - x.max(axis=1, keepdims=True))
    dense[rows] = (x / x.sum(axis=1, keepdims=True)) @ v64
    sparse = ora.sparse_branch(q64, k64, v64, crit, q_blocks=qb)
    e_pisa = rel_l2(to64(o)[0, 0][rows], dense[rows])
    e_sparse = rel_l2(sparse[rows], dense[rows])
    _say(f"[pisa vs dense seq8k head 0] rel L2: piecewise {e_pisa:.3e}, exact-only {e_sparse:.3e}")
    assert e_pisa < e_sparse


@pytest.mark.timeout(900)
def test_forward_pisa_parity_max_rows():
    # 4096 KV blocks: 64 pseudo-blocks of centroids, a full exclusion bitmask
    w = make_custom(1, 1, 64 * 4096 - 5, 64, dtype="bf16", kind="fourier1d", seed=100, k_crit=3,
                    k_marg=0)
    _pisa_check(w, 3, n_sample=12)


@pytest.mark.timeout(900)
def test_forward_pisa_parity_video75k():
    # every head, 32 sampled query blocks each (the last one included)
    w = make_workload("video75k")
    _pisa_check(w, w.k_crit, n_sample=32)
