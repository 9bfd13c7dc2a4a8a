"""Plain fp64 reference of the sparse-linear attention backward pass (test infrastructure only).

Gradients of the forward in ``oracle.sla`` with respect to Q, K, V and the
per-head mixing weight alpha, for fixed block index lists (the router's hard
top-k has no gradient; its lists are inputs here, as they are to the
forward).  SLA abstract: the kernel supports both the forward and the
backward pass, which fine-tuning needs.  Each function is the chain rule
written out over one step of the forward, in the forward's notation:

* mix (SLA2 technical summary, section 2.A equation): O = alpha O_s +
  (1 - alpha) O_l, so dO_s = alpha dO, dO_l = (1 - alpha) dO and
  dalpha = sum over rows and dims of dO * (O_s - O_l);
* sparse branch (SLA abstract; SLA2 summary section 1 item 1): per query
  row, P = softmax over the critical keys of q k^T / sqrt(d) and
  O_s = P V, so dV += P^T dO_s, dP = dO_s V^T,
  dS = P * (dP - rowsum(dO_s * O_s)), dq = dS K / sqrt(d),
  dK += dS^T q / sqrt(d);
* linear branch (SLA2 summary section 2.A): with f = phi(q),
  S_i = sum over the marginal blocks of H_j, sigma_i = sum of z_j,
  O_l = (f S_i) / (f . sigma_i): dnum = dO_l / den,
  dden = -(dO_l . O_l) / den, df = dnum S_i^T + dden sigma_i,
  dS_i = f^T dnum, dsigma_i = f^T dden; every marginal block j of query
  block i receives dH_j += dS_i, dz_j += dsigma_i; through
  H_j = phi(K_j)^T V_j and z_j = colsum phi(K_j):
  dphi(k_n) = dH_j v_n + dz_j, dv_n += phi(k_n) dH_j;
* phi = softmax over the features: dx = phi * (dphi - (dphi . phi)).

Pinned by central finite differences of the forward on tiny inputs (every
gradient, including alpha), by the alpha endpoints (alpha = 1 leaves only the
sparse branch, alpha = 0 only the linear one), and by the identity that the
softmax Jacobian annihilates constant shifts of the logits.
"""
from __future__ import annotations

import math

import numpy as np

from . import sla

BLOCK = sla.BLOCK


def phi_backward(f: np.ndarray, df: np.ndarray) -> np.ndarray:
    """Input gradient of the feature softmax f = phi(x): f * (df - rowsum(df * f))."""
    return f * (df - (df * f).sum(axis=-1, keepdims=True))


def sparse_branch_backward(q, k, v, crit_idx, do_s, block: int = BLOCK):
    """(dq, dk, dv) of O_s = softmax(q k^T / sqrt(d)) V over each query block's critical keys."""
    n, d = q.shape
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i, (a, b) in enumerate(sla.block_ranges(n, block)):
        c = crit_idx[i]
        if len(c) == 0:
            continue
        toks = np.concatenate([np.arange(*sla.block_ranges(n, block)[j]) for j in c])
        x = q[a:b] @ k[toks].T * scale
        p = np.exp(x - x.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v[toks]
        g = do_s[a:b]
        dv[toks] += p.T @ g
        dp = g @ v[toks].T
        ds = p * (dp - (g * o).sum(axis=1, keepdims=True))
        dq[a:b] += ds @ k[toks] * scale
        dk[toks] += ds.T @ q[a:b] * scale
    return dq, dk, dv


def linear_branch_backward(q, k, v, marg_idx, do_l, block: int = BLOCK):
    """(dq, dk, dv) of O_l = phi(q) S_i / (phi(q) . sigma_i) through H_j and z_j."""
    n, d = q.shape
    fk = sla.phi(k)
    H, z = sla.linear_states(k, v, block)
    dH = np.zeros_like(H)
    dz = np.zeros_like(z)
    dq = np.zeros_like(q)
    ranges = sla.block_ranges(n, block)
    for i, (a, b) in enumerate(ranges):
        m = marg_idx[i]
        if len(m) == 0:
            continue
        f = sla.phi(q[a:b])
        S = H[m].sum(axis=0)                 # [a][c]
        sig = z[m].sum(axis=0)
        num = f @ S
        den = f @ sig
        o_l = num / den[:, None]
        g = do_l[a:b]
        dnum = g / den[:, None]
        dden = -(g * o_l).sum(axis=1) / den
        df = dnum @ S.T + dden[:, None] * sig[None, :]
        dq[a:b] = phi_backward(f, df)
        dS = f.T @ dnum
        dsig = f.T @ dden
        for j in m:
            dH[j] += dS
            dz[j] += dsig
    dfk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for j, (a, b) in enumerate(ranges):
        dfk[a:b] = v[a:b] @ dH[j].T + dz[j][None, :]
        dv[a:b] = fk[a:b] @ dH[j]
    dk = phi_backward(fk, dfk)
    return dq, dk, dv


def backward_head(q, k, v, crit_idx, marg_idx, alpha: float, do, block: int = BLOCK):
    """(dq, dk, dv, dalpha) of O = alpha O_s + (1 - alpha) O_l for one head."""
    H, z = sla.linear_states(k, v, block)
    _, o_s, o_l = sla.forward_head(q, k, v, crit_idx, marg_idx, H, z, alpha, block)
    dqs, dks, dvs = sparse_branch_backward(q, k, v, crit_idx, alpha * do, block)
    dql, dkl, dvl = linear_branch_backward(q, k, v, marg_idx, (1.0 - alpha) * do, block)
    dalpha = float((do * (o_s - o_l)).sum())
    return dqs + dql, dks + dkl, dvs + dvl, dalpha
