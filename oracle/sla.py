"""Plain fp64 reference of the sparse-linear attention forward pass.

Test infrastructure only (see the package docstring).  Every function works
on float64 numpy arrays; per-head functions take ``[N, d]`` arrays and the
``*_batched`` wrappers loop over ``[B, H]``.  Nothing here is blocked, fused
or reordered beyond what each step's definition states: the sparse branch is
computed one-shot over the gathered critical tokens (no online softmax), and
the linear branch sums the per-block states before applying phi(Q).

Notation: N tokens, d features, block size ``block`` (64 by default), blocks
of ``block`` consecutive tokens, the last one possibly shorter (n_j valid
tokens).  nq = nkb = ceil(N / block).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

BLOCK = 64

CLASS_NEGLIGIBLE = 0
CLASS_MARGINAL = 1
CLASS_CRITICAL = 2


def n_blocks(n: int, block: int = BLOCK) -> int:
    return (n + block - 1) // block


def block_ranges(n: int, block: int = BLOCK):
    """[(start, stop)] of each block; the last block keeps only its valid tokens."""
    return [(j * block, min((j + 1) * block, n)) for j in range(n_blocks(n, block))]


# --------------------------------------------------------------------------
# Router (SLA2 summary, section 2.B: pooled Q and K, hard top-k at inference;
# SLA abstract: three classes of attention weights)
# --------------------------------------------------------------------------

def pool(x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Mean of each block of consecutive rows: [N, d] -> [nb, d].

    The router pools adjacent tokens (SLA2 summary, section 2.B); the mean
    over the n_j valid rows of block j is the reading taken, so a short tail
    block divides by n_j.
    Pinned by: constant blocks pool to themselves (tails included),
    linearity, brute-force loops.
    """
    n, d = x.shape
    out = np.empty((n_blocks(n, block), d), dtype=np.float64)
    for j, (a, b) in enumerate(block_ranges(n, block)):
        out[j] = x[a:b].sum(axis=0) / (b - a)
    return out


def block_logits(q_pool: np.ndarray, k_pool: np.ndarray) -> np.ndarray:
    """Block score logits s_ij = qbar_i . kbar_j / sqrt(d).

    The block-score map is softmax_j(s_ij) (SLA2 summary, section 2.B, with
    identity router projections); softmax is monotone along j, so ranking is
    done on the logits.
    Pinned by: brute-force loops; ranking equality with scipy's softmax.
    """
    d = q_pool.shape[1]
    return (q_pool @ k_pool.T) / math.sqrt(d)


def select(logits: np.ndarray, k_crit: int, k_marg: int):
    """Hard top-k split of each row of ``logits`` into three classes.

    Per row i, KV blocks are ordered by descending logit, equal logits by
    ascending block index; the first k_crit are critical, the next k_marg
    marginal, the rest negligible (SLA abstract; SLA2 summary, section 2.B
    hard top-k).  Returns (crit_idx [nq, k_crit], marg_idx [nq, k_marg],
    class_map [nq, nkb] int8), index lists ascending.
    Pinned by: brute-force sort on tiny rows; class counts; disjoint cover.
    """
    nq, nkb = logits.shape
    if not (0 <= k_crit and 0 <= k_marg and k_crit + k_marg <= nkb):
        raise ValueError("need 0 <= k_crit, k_marg and k_crit + k_marg <= nkb")
    # stable sort of -s keeps ascending j among equal logits
    order = np.argsort(-logits, axis=1, kind="stable")
    crit = np.sort(order[:, :k_crit], axis=1).astype(np.int64)
    marg = np.sort(order[:, k_crit:k_crit + k_marg], axis=1).astype(np.int64)
    cls = np.zeros((nq, nkb), dtype=np.int8)
    rows = np.arange(nq)[:, None]
    cls[rows, marg] = CLASS_MARGINAL
    cls[rows, crit] = CLASS_CRITICAL
    return crit, marg, cls


def route(q: np.ndarray, k: np.ndarray, k_crit: int, k_marg: int,
          block: int = BLOCK) -> Dict[str, np.ndarray]:
    """Pool, score and split one head: returns the index lists and intermediates."""
    qp = pool(q, block)
    kp = pool(k, block)
    s = block_logits(qp, kp)
    crit, marg, cls = select(s, k_crit, k_marg)
    return dict(pooled_q=qp, pooled_k=kp, logits=s, crit_idx=crit, marg_idx=marg,
                block_class=cls)


# --------------------------------------------------------------------------
# Linear branch states (PISA summary, per-block first-order matrices H_j;
# SPLA summary, section 2.2 compact linear-attention state)
# --------------------------------------------------------------------------

def phi(x: np.ndarray) -> np.ndarray:
    """Feature map: softmax over the feature (last) axis of each row."""
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def linear_states(k: np.ndarray, v: np.ndarray, block: int = BLOCK):
    """Per-block states H_j = phi(K_j)^T V_j ([d, d]) and z_j = column sums of phi(K_j).

    Pinned by: sum_a z_j[a] = n_j; column sums of H_j = sum of V_j rows;
    constant key rows give H_j = (1/d) 1 (sum V_j)^T; brute force.
    """
    n, d = k.shape
    fk = phi(k)
    nb = n_blocks(n, block)
    H = np.empty((nb, d, v.shape[1]), dtype=np.float64)
    z = np.empty((nb, d), dtype=np.float64)
    for j, (a, b) in enumerate(block_ranges(n, block)):
        H[j] = fk[a:b].T @ v[a:b]
        z[j] = fk[a:b].sum(axis=0)
    return H, z


# --------------------------------------------------------------------------
# Forward branches (SLA abstract; SLA2 summary sections 1 and 2.A)
# --------------------------------------------------------------------------

def _block_tokens(blocks: Sequence[int], n: int, block: int) -> np.ndarray:
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(j * block, min((j + 1) * block, n)) for j in blocks])


def sparse_branch(q: np.ndarray, k: np.ndarray, v: np.ndarray, crit_idx: np.ndarray,
                  block: int = BLOCK, q_blocks: Optional[Sequence[int]] = None) -> np.ndarray:
    """Exact softmax attention of each query block over its critical tokens only.

    Scores are q_t . k_n / sqrt(d); the softmax is renormalised over the
    critical keys of the row's query block (SLA2 summary, section 1 item 1).
    A query block with no critical block gets 0.  Computed one-shot: gather
    the critical tokens, then softmax, then the weighted sum of V.
    ``q_blocks`` restricts the work to some query blocks (other rows stay 0).
    Pinned by: all-critical routing equals dense attention (two independent
    routes: an N x N formula and torch's CPU scaled_dot_product_attention in
    float64); Q = 0 gives the mean of V over the critical tokens; per-token
    brute force.
    """
    n, d = q.shape
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    ranges = block_ranges(n, block)
    todo = range(len(ranges)) if q_blocks is None else q_blocks
    for i in todo:
        a, b = ranges[i]
        toks = _block_tokens(crit_idx[i], n, block)
        if toks.size == 0:
            continue
        s = (q[a:b] @ k[toks].T) / math.sqrt(d)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[a:b] = (p @ v[toks]) / p.sum(axis=1, keepdims=True)
    return out


def linear_branch(q: np.ndarray, H: np.ndarray, z: np.ndarray, marg_idx: np.ndarray,
                  block: int = BLOCK, q_blocks: Optional[Sequence[int]] = None) -> np.ndarray:
    """Linear attention of each query block through its marginal blocks' states.

    O_l[t] = phi(q_t) (sum_{j in M_i} H_j) / (phi(q_t) . sum_{j in M_i} z_j);
    a query block with no marginal block gets 0.
    Pinned by: all-marginal routing equals the quadratic form
    phi(Q) phi(K)^T V / (phi(Q) phi(K)^T 1); a uniform phi(q) gives the mean
    of V over the marginal tokens; exp(q - max q) in place of phi(q) gives
    the same result.
    """
    n, d = q.shape
    out = np.zeros((n, H.shape[2]), dtype=np.float64)
    fq = phi(q)
    ranges = block_ranges(n, block)
    todo = range(len(ranges)) if q_blocks is None else q_blocks
    for i in todo:
        a, b = ranges[i]
        m = marg_idx[i]
        if len(m) == 0:
            continue
        S = H[m].sum(axis=0)
        sig = z[m].sum(axis=0)
        out[a:b] = (fq[a:b] @ S) / (fq[a:b] @ sig)[:, None]
    return out


def mix(o_s: np.ndarray, o_l: np.ndarray, alpha: float) -> np.ndarray:
    """O = alpha O_s + (1 - alpha) O_l (SLA2 summary, section 2.A equation).

    Pinned by: alpha = 1 and alpha = 0 give the branches; affinity in alpha.
    """
    return alpha * o_s + (1.0 - alpha) * o_l


def forward_head(q, k, v, crit_idx, marg_idx, H, z, alpha, block=BLOCK, q_blocks=None):
    o_s = sparse_branch(q, k, v, crit_idx, block, q_blocks)
    o_l = linear_branch(q, H, z, marg_idx, block, q_blocks)
    return mix(o_s, o_l, alpha), o_s, o_l


def attention_head(q, k, v, alpha, k_crit, k_marg, block=BLOCK):
    """Route + states + forward for one head; returns a dict of every stage."""
    r = route(q, k, k_crit, k_marg, block)
    H, z = linear_states(k, v, block)
    o, o_s, o_l = forward_head(q, k, v, r["crit_idx"], r["marg_idx"], H, z, alpha, block)
    r.update(H=H, z=z, o=o, o_sparse=o_s, o_linear=o_l)
    return r


# --------------------------------------------------------------------------
# [B, H, N, d] wrappers
# --------------------------------------------------------------------------

def route_batched(q, k, k_crit, k_marg, block=BLOCK):
    B, Hh = q.shape[:2]
    outs = [[route(q[b, h], k[b, h], k_crit, k_marg, block) for h in range(Hh)]
            for b in range(B)]
    return {key: np.stack([np.stack([outs[b][h][key] for h in range(Hh)]) for b in range(B)])
            for key in outs[0][0]}


def linear_states_batched(k, v, block=BLOCK):
    B, Hh = k.shape[:2]
    Hs, zs = [], []
    for b in range(B):
        hb, zb = zip(*[linear_states(k[b, h], v[b, h], block) for h in range(Hh)])
        Hs.append(np.stack(hb))
        zs.append(np.stack(zb))
    return np.stack(Hs), np.stack(zs)


def forward_batched(q, k, v, crit_idx, marg_idx, H, z, alpha, block=BLOCK):
    """Returns (O, O_s, O_l), each [B, H, N, d], for given routing and states."""
    B, Hh = q.shape[:2]
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    o_s = np.zeros_like(o)
    o_l = np.zeros_like(o)
    for b in range(B):
        for h in range(Hh):
            o[b, h], o_s[b, h], o_l[b, h] = forward_head(
                q[b, h], k[b, h], v[b, h], crit_idx[b, h], marg_idx[b, h], H[b, h],
                z[b, h], float(alpha[h]), block)
    return o, o_s, o_l


def attention_batched(q, k, v, alpha, k_crit, k_marg, block=BLOCK):
    r = route_batched(q, k, k_crit, k_marg, block)
    H, z = linear_states_batched(k, v, block)
    o, o_s, o_l = forward_batched(q, k, v, r["crit_idx"], r["marg_idx"], H, z, alpha, block)
    r.update(H=H, z=z, o=o, o_sparse=o_s, o_linear=o_l)
    return r
