"""Covariance-aware routing of piecewise attention on the GPU against the
fp64 oracle (oracle/pisa.py, route_pisa).

Same bar as the plain router: masks bit-exact, disagreements excused only at
a class boundary where the oracle's covariance-aware logits tie within
1e-5; pooled means bit-exact for bf16 inputs; the block deviations M_j and
the logits within float32 rounding of the oracle's float64 values.  The
piecewise forward is then run on the GPU's covariance-aware lists, from the
statistics that the routing call leaves in its workspace, against the oracle
under the same lists (relative L2 <= 1e-2, max-abs <= 2e-2).
"""
import numpy as np
import pytest
import torch

from oracle import pisa as opisa
from oracle import sla as ora
from tests.parity_utils import (MAX_ABS_BF16, REL_L2_BF16, check_index_lists, classes_from_lists,
                                compare_classes, max_abs, rel_l2, to64)
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _s():
    import block_sparse_linear_route_amd as s
    return s


def _say(msg):
    print(msg, flush=True)


def _route_pisa_check(w, heads=None, fwd_blocks=None, seed=0):
    s = _s()
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    B, H, N, d = w.shape
    nkb = ora.n_blocks(N)
    r = s.route_pisa(q, k, v, w.k_crit, w.k_marg, want_class=True, want_logits=True,
                     want_pooled=True, want_dev=True)
    o = s.forward_attend_pisa(q, k, v, r["crit_idx"], r["_workspace"])
    torch.cuda.synchronize()
    q64, k64, v64 = to64(w.q), to64(w.k), to64(w.v)
    exc = unexc = rows = 0
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    rng = np.random.default_rng(seed)
    dev_err = 0.0
    got_o, ref_o = [], []
    og = to64(o)
    for b, h in heads:
        ro = opisa.route_pisa(q64[b, h], k64[b, h], v64[b, h], w.k_crit, w.k_marg)
        crit = r["crit_idx"][b, h].cpu().numpy()
        marg = r["marg_idx"][b, h].cpu().numpy()
        assert crit.shape == (nkb, w.k_crit) and marg.shape == (nkb, w.k_marg)
        check_index_lists(crit, marg, nkb)
        cls = r["block_class"][b, h].cpu().numpy()
        np.testing.assert_array_equal(cls, classes_from_lists(crit, marg, nkb))
        e, u, rr = compare_classes(cls, ro["block_class"], ro["logits"], w.k_crit, w.k_marg)
        exc, unexc, rows = exc + e, unexc + u, rows + rr
        if w.q.dtype == torch.bfloat16:
            np.testing.assert_array_equal(r["pooled_q"][b, h].cpu().numpy(),
                                          ro["pooled_q"].astype(np.float32))
        mg = r["block_dev"][b, h].cpu().numpy().astype(np.float64)
        dev_err = max(dev_err, float(np.max(np.abs(mg - ro["block_dev"]) / ro["block_dev"].max())))
        np.testing.assert_allclose(mg, ro["block_dev"], rtol=2e-6, atol=1e-6 * ro["block_dev"].max())
        np.testing.assert_allclose(r["block_logits"][b, h].cpu().numpy(), ro["logits"],
                                   rtol=1e-6, atol=1e-6)
        # the piecewise forward on the GPU's own covariance-aware lists
        nb = nkb
        qb = list(range(nb)) if fwd_blocks is None or fwd_blocks >= nb else \
            sorted(set(rng.choice(nb - 1, fwd_blocks - 1, replace=False).tolist()) | {nb - 1})
        ref, _, _ = opisa.pisa_head(q64[b, h], k64[b, h], v64[b, h], crit.astype(np.int64), q_blocks=qb)
        rws = np.concatenate([np.arange(64 * i, min(64 * i + 64, N)) for i in qb])
        got_o.append(og[b, h][rws])
        ref_o.append(ref[rws])
    a, bb = np.concatenate(got_o), np.concatenate(ref_o)
    e_o, m_o = rel_l2(a, bb), max_abs(a, bb)
    _say(f"[pisa route {w.name} N={N} d={d} kc={w.k_crit} km={w.k_marg} {w.q.dtype}; {len(heads)} heads] "
         f"excused ties {exc} (rows {rows}), unexcused {unexc}; M_j max rel err {dev_err:.1e}; "
         f"forward relL2 {e_o:.2e} maxabs {m_o:.2e}")
    assert unexc == 0
    assert e_o <= REL_L2_BF16 and m_o <= MAX_ABS_BF16
    return r


@pytest.mark.parametrize("name", ["tiny", "seq8k"])
def test_route_pisa_parity(name):
    _route_pisa_check(make_workload(name))


@pytest.mark.timeout(900)
def test_route_pisa_parity_video32k():
    _route_pisa_check(make_workload("video32k"), fwd_blocks=64)


@pytest.mark.parametrize("N,d,dtype,kc,km,H,seed", [
    (65, 128, "bf16", 1, 1, 2, 120),            # a one-token last block
    (1000, 64, "bf16", 3, 5, 2, 121),
    (777, 128, "fp32", 2, 4, 1, 122),
    (4095, 128, "bf16", 0, 64, 1, 123),         # no critical block
    (8190, 64, "fp32", 128, 0, 1, 124),         # every block critical
    (64 * 300 + 17, 128, "bf16", 65, 30, 1, 125),
])
def test_route_pisa_parity_shapes(N, d, dtype, kc, km, H, seed):
    w = make_custom(1, H, N, d, dtype=dtype, kind="fourier1d", seed=seed, k_crit=kc, k_marg=km)
    _route_pisa_check(w, fwd_blocks=24)


@pytest.mark.timeout(900)
def test_route_pisa_parity_long_rows():
    # 4096 KV blocks: two rows per selection workgroup
    w = make_custom(1, 1, 64 * 4096 - 5, 64, dtype="bf16", kind="fourier1d", seed=126, k_crit=40,
                    k_marg=80)
    _route_pisa_check(w, fwd_blocks=8)


@pytest.mark.timeout(900)
def test_route_pisa_parity_video75k():
    _route_pisa_check(make_workload("video75k"), fwd_blocks=8)


def test_route_pisa_workspace_serves_the_forward():
    # the statistics the routing call leaves in its workspace are those of
    # sla_pisa_statistics: the forward from them equals sla_forward_pisa
    s = _s()
    w = make_custom(1, 2, 3000, 128, seed=127, k_crit=5, k_marg=9)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    r = s.route_pisa(q, k, v, 5, 9)
    o1 = s.forward_attend_pisa(q, k, v, r["crit_idx"], r["_workspace"])
    o2 = s.forward_pisa(q, k, v, r["crit_idx"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
