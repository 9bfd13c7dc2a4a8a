"""Backward pass on the GPU against the fp64 oracle (oracle/backward.py).

The GPU's own router lists are used on both sides (the lists carry no
gradient).  P, dS, the linear-branch operands and dH enter the matrix cores
as bf16 (relative rounding 2^-9 each, a few such roundings chained along
every gradient path) with float32 accumulation, so the bar is relative L2
<= 2e-2 and max-abs <= 5e-2 of the gradient's largest magnitude, per
gradient.  dalpha = sum dO * (O_s - O_l) inherits the forward's error: by
Cauchy-Schwarz |error| <= ||dO|| * ||error of (O_s - O_l)||, and the branch
outputs meet the forward's 1e-2 relative L2 bar, so dalpha is held to
1e-2 * ||dO|| * ||O_s - O_l|| (both norms from the oracle, per head).
"""
import numpy as np
import pytest
import torch

from oracle import backward as obwd
from oracle import sla as ora
from tests.parity_utils import max_abs, rel_l2, to64
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REL_L2_GRAD = 2e-2
MAX_ABS_GRAD = 5e-2


def _s():
    import block_sparse_linear_route_amd as s
    return s


def _say(msg):
    print(msg, flush=True)


def _bwd_check(w, heads=None, seed=0):
    s = _s()
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    B, H, N, d = w.shape
    g = torch.Generator().manual_seed(1000 + seed)
    do = torch.randn(B, H, N, d, generator=g).to(w.q.dtype).to(DEV)
    r = s.route(q, k, w.k_crit, w.k_marg)
    Hs, zs = s.linear_states(k, v)
    dq, dk, dv, da = s.backward(q, k, v, do, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha)
    torch.cuda.synchronize()
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    q64, k64, v64, do64 = to64(w.q), to64(w.k), to64(w.v), to64(do.cpu())
    res = {"dq": [], "dk": [], "dv": []}
    da_ref = np.zeros(H)
    da_tol = np.zeros(H)
    for b, h in heads:
        crit = r["crit_idx"][b, h].cpu().numpy().astype(np.int64)
        marg = r["marg_idx"][b, h].cpu().numpy().astype(np.int64)
        gq, gk, gv, ga = obwd.backward_head(q64[b, h], k64[b, h], v64[b, h], crit, marg,
                                            float(w.alpha[h]), do64[b, h])
        H64, z64 = ora.linear_states(k64[b, h], v64[b, h])
        _, os_, ol_ = ora.forward_head(q64[b, h], k64[b, h], v64[b, h], crit, marg, H64, z64,
                                       float(w.alpha[h]))
        da_ref[h] += ga
        da_tol[h] += 1e-2 * np.linalg.norm(do64[b, h]) * np.linalg.norm(os_ - ol_)
        for key, got, ref in (("dq", dq, gq), ("dk", dk, gk), ("dv", dv, gv)):
            res[key].append((got[b, h].cpu().numpy().astype(np.float64), ref))
    msg, fails = [], []
    for key, pairs in res.items():
        a = np.concatenate([p[0] for p in pairs])
        bb = np.concatenate([p[1] for p in pairs])
        e, m, sc = rel_l2(a, bb), max_abs(a, bb), float(np.abs(bb).max())
        msg.append(f"{key}: relL2 {e:.2e} maxabs {m:.2e} (max {sc:.2e})")
        if e > REL_L2_GRAD or m > MAX_ABS_GRAD * max(sc, 1e-6):
            fails.append(key)
    for h in sorted({h for _, h in heads}):
        got = float(da[h].cpu())
        msg.append(f"dalpha[{h}] {got:.6g} ref {da_ref[h]:.6g} (bound {da_tol[h]:.2e})")
        if B == 1 and abs(got - da_ref[h]) > da_tol[h]:
            fails.append(f"dalpha[{h}]")
    _say(f"[backward {w.name} N={N} d={d} kc={w.k_crit} km={w.k_marg}] " + " ".join(msg))
    assert not fails, fails


@pytest.mark.parametrize("N,d,kc,km,H,seed", [
    (1000, 128, 3, 5, 2, 90),
    (777, 64, 2, 4, 2, 91),
    (4095, 128, 6, 9, 1, 92),
    (65, 128, 1, 1, 2, 93),        # two blocks, the second one row long
    (1000, 128, 0, 6, 1, 94),      # linear branch only
    (1000, 128, 7, 0, 1, 95),      # sparse branch only
    (1000, 128, 16, 0, 1, 96),     # every block critical: dense attention
    # critical lists past the 64 entries one list register holds (forward
    # recompute and the query-major dQ kernel refill them every 64 steps)
    (300 * 64 + 17, 128, 64, 10, 1, 110),
    (300 * 64 + 17, 128, 65, 20, 1, 111),
    (300 * 64 + 17, 128, 129, 30, 1, 112),
    (270 * 64, 64, 200, 30, 1, 113),
])
def test_backward_parity_shapes(N, d, kc, km, H, seed):
    w = make_custom(1, H, N, d, dtype="bf16", kind="fourier1d", seed=seed, k_crit=kc, k_marg=km)
    _bwd_check(w, seed=seed)


@pytest.mark.parametrize("name,heads", [("seq8k", [(0, 0), (0, 9)]), ("video32k", [(0, 4)])])
def test_backward_parity_workloads(name, heads):
    _bwd_check(make_workload(name), heads)


def test_backward_is_deterministic():
    s = _s()
    w = make_custom(1, 2, 3000, 128, seed=97, k_crit=5, k_marg=9)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    do = torch.randn_like(w.q.float()).bfloat16().to(DEV)
    r = s.route(q, k, 5, 9)
    Hs, zs = s.linear_states(k, v)
    a = s.backward(q, k, v, do, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha)
    b = s.backward(q, k, v, do, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("kc,km", [(5, 9), (0, 7), (6, 0)])
def test_saved_forward_and_backward_equal_the_one_call_backward(kc, km):
    # sla_backward is sla_forward_save followed by sla_backward_saved: the
    # split gives the same bits, O equals sla_forward's, and the saved
    # workspace serves a second backward with another dO
    s = _s()
    w = make_custom(1, 2, 3000, 128, seed=101 + kc, k_crit=kc, k_marg=km)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    r = s.route(q, k, kc, km)
    Hs, zs = s.linear_states(k, v)
    o_ref = s.forward(q, k, v, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha)
    o, ws = s.forward_save(q, k, v, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha)
    torch.cuda.synchronize()
    _say(f"[saved kc={kc} km={km}] max|O - forward O| {float((o.float() - o_ref.float()).abs().max()):.3e}")
    assert torch.equal(o, o_ref)
    for seed in (0, 1):
        g = torch.Generator().manual_seed(seed)
        do = torch.randn(w.q.shape, generator=g).bfloat16().to(DEV)
        got = s.backward_saved(q, k, v, do, r["crit_idx"], r["marg_idx"], w.alpha, ws)
        ref = s.backward(q, k, v, do, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha)
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv", "dalpha"), got, ref):
            assert torch.equal(x, y), name


def test_dalpha_is_the_sum_over_the_forward_branches():
    # dalpha_h = sum over batch, rows and dims of dO * (O_s - O_l), with the
    # branch outputs the forward itself writes: a float32 reduction of the
    # same numbers, to 1e-5 relative
    s = _s()
    w = make_custom(2, 3, 2000, 128, seed=98, k_crit=4, k_marg=8)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    do = torch.randn_like(w.q.float()).bfloat16().to(DEV)
    r = s.route(q, k, 4, 8)
    Hs, zs = s.linear_states(k, v)
    _, o_s, o_l = s.forward(q, k, v, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha, branches=True)
    _, _, _, da = s.backward(q, k, v, do, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha)
    torch.cuda.synchronize()
    ref = (do.double() * (o_s.double() - o_l.double())).sum(dim=(0, 2, 3)).cpu().numpy()
    got = da.double().cpu().numpy()
    _say(f"[dalpha sum] got {got} ref {ref}")
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-3)


@pytest.mark.timeout(900)
def test_backward_parity_max_rows():
    # 4096 KV blocks: 128 bit words per transposed row, lists up to 4096 long
    # (checked on sampled rows of one head against the oracle's full head)
    w = make_custom(1, 1, 64 * 4096 - 5, 64, dtype="bf16", kind="fourier1d", seed=99, k_crit=3,
                    k_marg=5)
    _bwd_check(w)
