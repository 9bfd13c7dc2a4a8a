"""fp8 forward paired with the bf16 backward (quantisation-aware training).

SLA2 technical summary, section 2.C: during training the forward runs the
sparse branch in a low-bit format while the backward stays in 16-bit.
sla_forward_save_fp8 runs the fp8 forward and keeps its O_s, O_l and
softmax normalisers; sla_backward_saved then rebuilds P from the bf16
scores and the fp8 normaliser and takes rowsum(dO_s * O_s) from the fp8
O_s.  The fp64 reference of that pairing is oracle/qat.py (its reading and
pins are stated there): the low-bit forward emulated on the E4M3 round trip
of Q, K and V, the rest the plain backward.  Checked here:

* the O that sla_forward_save_fp8 writes equals sla_forward_fp8's bit for
  bit, and the saved statistics are reproducible (a second save gives
  bit-identical gradients);
* dk and dv against oracle/qat.py at the bf16 backward's bar, relative L2
  <= 2e-2 (the saved statistics enter them only through P and dS);
* dq against oracle/qat.py within the bf16 bar plus what the fp8 forward's
  own error can add.  The GPU's fp8 forward also rounds P to E4M3 inside its
  PV product, which the emulation leaves out, so its O_s differs from the
  emulated O^q_s; the row term D_i = rowsum(dO_s * O_s) then moves by
  delta_i, dS by -P delta_i and dq_i by -delta_i kbar_i / sqrt(d) with kbar_i
  the P-weighted key mean.  With ||O_s - O^q_s||_F <= 5e-2 ||O^q_s||_F (the
  fp8 branch's output bar) and Cauchy-Schwarz per row:
      ||dq error||_F <= 2e-2 ||dq|| + alpha max_i ||dO_i|| 5e-2 ||O^q_s||_F
                        max_i ||kbar_i|| / sqrt(d)
  (every quantity from the oracle).  dq is the gradient this pairing moves
  most: D_i enters every key of the row with the same sign;
* dalpha = sum dO (O_s - O_l) within 5e-2 ||dO|| ||O^q_s - O_l|| per head
  (Cauchy-Schwarz with the fp8 bar on the branch outputs).
The distance to the exact gradients of the unquantised forward
(oracle/backward.py) is printed for reference only.
"""
import numpy as np
import pytest
import torch

from oracle import backward as obwd
from oracle import qat as oqat
from oracle import sla as ora
from tests.parity_utils import rel_l2, to64
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REL_L2_FP8 = 5e-2
REL_L2_GRAD = 2e-2


def _kbar_max(q, k, crit, block=64):
    """max over rows of the norm of the softmax-weighted mean of the row's
    critical keys (oracle inputs, fp64)."""
    n, d = q.shape
    best = 0.0
    for i, (a, b) in enumerate(ora.block_ranges(n, block)):
        toks = ora._block_tokens(crit[i], n, block)
        if toks.size == 0:
            continue
        sc = q[a:b] @ k[toks].T / np.sqrt(d)
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        best = max(best, float(np.linalg.norm(p @ k[toks], axis=1).max()))
    return best


def _s():
    import block_sparse_linear_route_amd as s
    return s


def _qat_setup(w, seed):
    s = _s()
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    g = torch.Generator().manual_seed(2000 + seed)
    do = torch.randn(w.shape, generator=g).to(w.q.dtype).to(DEV)
    r = s.route_quantize(q, k, w.k_crit, w.k_marg)
    Hs, zs, v8, vs = s.linear_states_quantize(k, v)
    codes = (r["q8"], r["q_scale"], r["k8"], r["k_scale"], v8, vs)
    return s, q, k, v, do, r, Hs, zs, codes


def test_saved_fp8_forward_equals_the_fp8_forward():
    w = make_custom(1, 2, 2000, 128, dtype="bf16", seed=61, k_crit=5, k_marg=9)
    s, q, k, v, do, r, Hs, zs, codes = _qat_setup(w, 0)
    o_ref, os_ref, ol_ref = s.forward_fp8(q, *codes, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha,
                                          branches=True)
    o, ws = s.forward_save_fp8(q, k, v, *codes, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    # the backward workspace holds O_s and O_l after the forward's workspace and
    # the O scratch; compare through the gradients instead of the layout: a
    # second save into the same workspace gives bit-identical gradients
    g1 = s.backward_saved(q, k, v, do, r["crit_idx"], r["marg_idx"], w.alpha, ws)
    s.forward_save_fp8(q, k, v, *codes, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha, workspace=ws)
    g2 = s.backward_saved(q, k, v, do, r["crit_idx"], r["marg_idx"], w.alpha, ws)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    assert torch.isfinite(os_ref).all() and torch.isfinite(ol_ref).all()


def _qat_check(w, heads=None, seed=0):
    s, q, k, v, do, r, Hs, zs, codes = _qat_setup(w, seed)
    o, ws = s.forward_save_fp8(q, k, v, *codes, r["crit_idx"], r["marg_idx"], Hs, zs, w.alpha)
    dq, dk, dv, da = s.backward_saved(q, k, v, do, r["crit_idx"], r["marg_idx"], w.alpha, ws)
    torch.cuda.synchronize()
    B, H, N, d = w.shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    q64, k64, v64, do64 = to64(w.q), to64(w.k), to64(w.v), to64(do.cpu())
    res = {"dq": [], "dk": [], "dv": []}
    msg, fails = [], []
    dq_extra = 0.0
    for b, h in heads:
        crit = r["crit_idx"][b, h].cpu().numpy().astype(np.int64)
        marg = r["marg_idx"][b, h].cpu().numpy().astype(np.int64)
        a_h = float(w.alpha[h])
        gq, gk, gv, ga = oqat.qat_backward_head(q64[b, h], k64[b, h], v64[b, h], crit, marg, a_h,
                                                do64[b, h])
        xq, xk, xv, _ = obwd.backward_head(q64[b, h], k64[b, h], v64[b, h], crit, marg, a_h,
                                           do64[b, h])
        osq, _ = oqat.sparse_forward_stats(oqat.fp8_round_trip(q64[b, h]),
                                           oqat.fp8_round_trip(k64[b, h]),
                                           oqat.fp8_round_trip(v64[b, h]), crit)
        H64, z64 = ora.linear_states(k64[b, h], v64[b, h])
        ol_ = ora.linear_branch(q64[b, h], H64, z64, marg)
        tol = REL_L2_FP8 * np.linalg.norm(do64[b, h]) * np.linalg.norm(osq - ol_)
        dq_extra += (a_h * float(np.linalg.norm(do64[b, h], axis=1).max()) * REL_L2_FP8
                     * float(np.linalg.norm(osq)) * _kbar_max(q64[b, h], k64[b, h], crit)
                     / np.sqrt(d)) ** 2
        if B == 1:
            got = float(da[h].cpu())
            msg.append(f"dalpha[{h}] {got:.6g} ref {ga:.6g} (bound {tol:.2e})")
            if abs(got - ga) > tol:
                fails.append(f"dalpha[{h}]")
        for key, got, ref, ex in (("dq", dq, gq, xq), ("dk", dk, gk, xk), ("dv", dv, gv, xv)):
            res[key].append((got[b, h].cpu().numpy().astype(np.float64), ref, ex))
    for key, pairs in res.items():
        a = np.concatenate([p[0] for p in pairs])
        bb = np.concatenate([p[1] for p in pairs])
        ex = np.concatenate([p[2] for p in pairs])
        e = rel_l2(a, bb)
        msg.append(f"{key}: relL2 {e:.2e} (to the unquantised gradient {rel_l2(a, ex):.2e})")
        if key == "dq":
            # the per-head bounds add in quadrature over the heads' rows
            bound = REL_L2_GRAD * np.linalg.norm(bb) + np.sqrt(dq_extra)
            msg.append(f"(dq error {np.linalg.norm(a - bb):.3g}, bound {bound:.3g})")
            if np.linalg.norm(a - bb) > bound:
                fails.append(key)
        elif e > REL_L2_GRAD:
            fails.append(key)
    print(f"[qat {w.name} N={N} kc={w.k_crit} km={w.k_marg}] " + " ".join(msg), flush=True)
    assert not fails, fails


@pytest.mark.parametrize("N,kc,km,H,seed", [
    (1000, 3, 5, 2, 70),          # ragged last block
    (4096, 10, 20, 2, 71),
    (300 * 64 + 17, 70, 30, 1, 72),   # critical list past 64 entries
])
def test_qat_gradients_shapes(N, kc, km, H, seed):
    _qat_check(make_custom(1, H, N, 128, dtype="bf16", seed=seed, k_crit=kc, k_marg=km), seed=seed)


def test_qat_gradients_seq8k():
    _qat_check(make_workload("seq8k"), heads=[(0, 0), (0, 9)], seed=3)
