"""Second-order routing score on the GPU against the fp64 oracle (oracle/taylor.py).

Same bar as the plain router: masks bit-exact, disagreements excused only at
a class boundary where the oracle logits tie within 1e-5; pooled means
bit-exact for bf16 inputs; block key variances and logits within float32
rounding of the oracle's float64 values.
"""
import numpy as np
import pytest
import torch

from oracle import sla as ora
from oracle import taylor as otay
from tests.parity_utils import check_index_lists, classes_from_lists, compare_classes, to64
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _s():
    import block_sparse_linear_route_amd as s
    return s


def _say(msg):
    print(msg, flush=True)


def _taylor_check(w, heads=None):
    s = _s()
    q, k = w.q.to(DEV), w.k.to(DEV)
    B, H, N, d = w.shape
    nkb = ora.n_blocks(N)
    r = s.route(q, k, w.k_crit, w.k_marg, want_class=True, want_logits=True, want_pooled=True,
                score="taylor")
    torch.cuda.synchronize()
    q64, k64 = to64(w.q), to64(w.k)
    exc = unexc = rows = 0
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        o = otay.route_taylor(q64[b, h], k64[b, h], w.k_crit, w.k_marg)
        crit = r["crit_idx"][b, h].cpu().numpy()
        marg = r["marg_idx"][b, h].cpu().numpy()
        assert crit.shape == (nkb, w.k_crit) and marg.shape == (nkb, w.k_marg)
        check_index_lists(crit, marg, nkb)
        cls = r["block_class"][b, h].cpu().numpy()
        np.testing.assert_array_equal(cls, classes_from_lists(crit, marg, nkb))
        e, u, rr = compare_classes(cls, o["block_class"], o["logits"], w.k_crit, w.k_marg)
        exc, unexc, rows = exc + e, unexc + u, rows + rr
        if w.q.dtype == torch.bfloat16:
            np.testing.assert_array_equal(r["pooled_k"][b, h].cpu().numpy(),
                                          o["pooled_k"].astype(np.float32))
        np.testing.assert_allclose(r["key_var"][b, h].cpu().numpy(), o["k_var"], rtol=1e-6,
                                   atol=1e-12)
        np.testing.assert_allclose(r["block_logits"][b, h].cpu().numpy(), o["logits"],
                                   rtol=1e-6, atol=1e-6)
    _say(f"[taylor route {w.name} N={N} d={d} kc={w.k_crit} km={w.k_marg}] excused ties {exc} "
         f"(rows {rows}), unexcused {unexc}")
    assert unexc == 0
    return r


@pytest.mark.parametrize("name,heads", [("tiny", None), ("seq8k", None),
                                        ("video32k", [(0, 0), (0, 6), (0, 11)])])
def test_taylor_route_parity(name, heads):
    _taylor_check(make_workload(name), heads)


@pytest.mark.parametrize("N,d,dtype,kc,km,H,seed", [
    (65, 128, "bf16", 1, 1, 2, 70), (127, 128, "bf16", 1, 0, 1, 71),
    (1000, 128, "bf16", 3, 5, 2, 72), (4095, 128, "bf16", 0, 64, 1, 73),
    (8190, 128, "bf16", 128, 0, 1, 74), (3000, 64, "fp32", 10, 37, 2, 75),
    (64 * 300 + 1, 128, "bf16", 30, 60, 1, 76),
])
def test_taylor_route_parity_shapes(N, d, dtype, kc, km, H, seed):
    w = make_custom(1, H, N, d, dtype=dtype, kind="fourier1d", seed=seed, k_crit=kc, k_marg=km)
    _taylor_check(w)


@pytest.mark.parametrize("nkb,kc,km", [(700, 30, 60), (2101, 26, 51), (4096, 40, 80)])
def test_taylor_route_parity_long_rows(nkb, kc, km):
    w = make_custom(1, 1, 64 * nkb - 3, 128, dtype="bf16", kind="fourier1d", seed=nkb + 1,
                    k_crit=kc, k_marg=km)
    _taylor_check(w)


def test_taylor_route_constant_key_blocks_equal_plain_route():
    # keys constant within each block: every variance is 0, so the split and
    # the logits are those of the plain router
    s = _s()
    g = torch.Generator().manual_seed(77)
    N, d = 64 * 40, 128
    q = torch.randn(1, 2, N, d, generator=g).bfloat16().to(DEV)
    kb = torch.randn(1, 2, 40, 1, d, generator=g).bfloat16()
    k = kb.expand(1, 2, 40, 64, d).reshape(1, 2, N, d).contiguous().to(DEV)
    a = s.route(q, k, 5, 9, want_logits=True, want_pooled=True, score="taylor")
    b = s.route(q, k, 5, 9, want_logits=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(a["key_var"]).item() == 0
    assert torch.equal(a["crit_idx"], b["crit_idx"]) and torch.equal(a["marg_idx"], b["marg_idx"])
    assert torch.equal(a["block_logits"], b["block_logits"])


def test_taylor_route_changes_the_split_on_the_workload():
    # the spread term matters: on the 8k-token workload some rows route
    # differently from the plain mean score (both sides checked above)
    s = _s()
    w = make_workload("seq8k")
    q, k = w.q.to(DEV), w.k.to(DEV)
    a = s.route(q, k, w.k_crit, w.k_marg, score="taylor")
    b = s.route(q, k, w.k_crit, w.k_marg)
    torch.cuda.synchronize()
    rows = (a["crit_idx"] != b["crit_idx"]).any(dim=-1) | (a["marg_idx"] != b["marg_idx"]).any(dim=-1)
    diff = rows.float().mean().item()
    _say(f"[taylor vs mean seq8k] rows with a different split: {diff:.3f}")
    assert diff > 0.0


@pytest.mark.timeout(900)
def test_taylor_route_parity_video75k():
    _taylor_check(make_workload("video75k"), heads=[(0, 0), (0, 21), (0, 39)])
