"""Quantisation-aware pairing of the low-bit forward with the 16-bit backward.

Test infrastructure only: nothing on the product path imports this module.

SLA2 technical summary, section 2.C: during training the forward runs the
sparse branch in a low-bit format while the backward stays in 16-bit, so the
model learns to live with the quantisation error.  The page gives no formula;
the reading taken here: the backward is the ordinary softmax backward of the
sparse branch on the unquantised Q, K, V, except for the two per-row
quantities that a recomputing backward takes from its forward instead of
recomputing them, the softmax normaliser and the output O_s, which come from
the low-bit forward.  With L_i the log-sum-exp of the low-bit forward's
scores over the critical keys and O^q_s its output:

    P = exp(q k^T / sqrt(d) - L_i) over the critical keys,
    dv += P^T dO_s,   dP = dO_s v^T,   dS = P * (dP - rowsum(dO_s * O^q_s)),
    dq += dS k / sqrt(d),   dk += dS^T q / sqrt(d),

the linear branch (not quantised) has its plain backward, and
dalpha = sum dO * (O^q_s - O_l).  The low-bit forward is emulated as the
fp64 sparse branch on the quantiser's round trip of Q, K and V (by default
oracle.fp8: per-block E4M3 codes, then their values); the rounding of P
inside a kernel's PV product is that kernel's own arithmetic and is not part
of the emulation.

Pinned (tests/test_oracle_pins_qat.py) by: the identity quantiser gives the
exact gradients of backward_head, which finite differences pin; quantising
V alone leaves dv exact and moves dq and dk by the closed form
-(P * rowsum(dO_s * (O^q_s - O_s))) k / sqrt(d) (and its transpose); the
saved-statistics backward fed the exact normaliser and output equals
sparse_branch_backward.
"""
from __future__ import annotations

import math

import numpy as np

from . import backward as obwd
from . import fp8 as ofp8
from . import sla

BLOCK = sla.BLOCK


def fp8_round_trip(x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Values of the per-block E4M3 codes of x (one head, [N, d])."""
    codes, scales = ofp8.quantize_blocks(np.asarray(x, dtype=np.float32), block)
    return ofp8.dequantize_blocks(codes, scales, block).astype(np.float64)


def sparse_forward_stats(q, k, v, crit_idx, block: int = BLOCK):
    """(O_s, L) of the sparse branch: output and natural-log normaliser per row
    (-inf and 0 for a query block without critical keys)."""
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    lse = np.full(n, -np.inf)
    for i, (a, b) in enumerate(sla.block_ranges(n, block)):
        toks = sla._block_tokens(crit_idx[i], n, block)
        if toks.size == 0:
            continue
        s = q[a:b] @ k[toks].T / math.sqrt(d)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        den = e.sum(axis=1, keepdims=True)
        o[a:b] = (e @ v[toks]) / den
        lse[a:b] = (m + np.log(den))[:, 0]
    return o, lse


def sparse_branch_backward_saved(q, k, v, crit_idx, do_s, o_s, lse, block: int = BLOCK):
    """(dq, dk, dv) of the sparse branch with P rebuilt from q k^T and the given
    normaliser L, and rowsum(dO_s * O_s) taken from the given O_s."""
    n, d = q.shape
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i, (a, b) in enumerate(sla.block_ranges(n, block)):
        toks = sla._block_tokens(crit_idx[i], n, block)
        if toks.size == 0:
            continue
        p = np.exp(q[a:b] @ k[toks].T * scale - lse[a:b, None])
        g = do_s[a:b]
        dv[toks] += p.T @ g
        dp = g @ v[toks].T
        ds = p * (dp - (g * o_s[a:b]).sum(axis=1, keepdims=True))
        dq[a:b] += ds @ k[toks] * scale
        dk[toks] += ds.T @ q[a:b] * scale
    return dq, dk, dv


def qat_backward_head(q, k, v, crit_idx, marg_idx, alpha: float, do, quant=fp8_round_trip,
                      block: int = BLOCK):
    """(dq, dk, dv, dalpha) of the low-bit-forward / 16-bit-backward pairing
    for one head; ``quant`` maps a [N, d] tensor to its quantised values."""
    qq, kq, vq = quant(q), quant(k), quant(v)
    o_sq, lse_q = sparse_forward_stats(qq, kq, vq, crit_idx, block)
    dqs, dks, dvs = sparse_branch_backward_saved(q, k, v, crit_idx, alpha * do, o_sq, lse_q, block)
    dql, dkl, dvl = obwd.linear_branch_backward(q, k, v, marg_idx, (1.0 - alpha) * do, block)
    H, z = sla.linear_states(k, v, block)
    o_l = sla.linear_branch(q, H, z, marg_idx, block)
    dalpha = float((do * (o_sq - o_l)).sum())
    return dqs + dql, dks + dkl, dvs + dvl, dalpha
