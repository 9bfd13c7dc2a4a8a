"""Plain fp64 reference of piecewise exact-or-approximate attention (test infrastructure only).

PISA technical summary ("PISA - Atención Dispersa por Tramos para
Transformers de Difusión Eficientes"), section 2, "Algoritmo Central": the
KV blocks of query block i are split into the selected set S_i, attended
exactly, and the rest U_i, whose softmax contribution is expanded around the
block centroid.  Every term goes into one softmax numerator N_t and one
denominator D_t, o_t = N_t / D_t:
* exact terms: sum over the tokens of S_i of exp(q_t . k_n) v_n (and exp(q_t . k_n) in D_t);
* zero-order terms per unselected block: alpha_{t,j} = exp(q_t . kbar_j)
  times the block's value sum (and times its token count n_j in D_t);
* one global first-order correction q_t Hbar sum_{j in U_i} alpha_{t,j},
  Hbar = mean over all KV blocks of the per-block first-order matrices.

Readings fixed here (each is listed in the design notes):
* q_t is the scaled query q_t / sqrt(d) throughout (standard scaled
  dot-product attention); the page writes the exponents without the scale;
* the first-order matrix of block j is the one the Taylor step produces,
  H_j = sum_n (k_n - kbar_j)^T v_n (d x d, [a][c]: key feature a, value dim c),
  kbar_j the mean of the block's valid keys;
* the first-order term of D_t is q_t . sum_n (k_n - kbar_j) = 0 exactly, so
  D_t has exact and zero-order terms only;
* S_i is the router's critical list; U_i is every other KV block.

Covariance-aware routing ("Enrutamiento Consciente de la Covarianza": the
selection score of a block takes in, beside its attention score, the norm
M_j = ||H_j - Hbar|| of its first-order matrix's deviation from the shared
Hbar, so that blocks of high relevance or high heterogeneity are computed
exactly) is ``route_pisa``.  Readings fixed here:
* an unselected block j replaces its own first-order term by Hbar, so N_t
  misses alpha_{t,j} (q_t / sqrt(d)) (H_j - Hbar), whose norm is at most
  alpha_{t,j} (|q_t| / sqrt(d)) M_j;
* the norm is the L2 norm of the matrix taken as a vector (Frobenius),
  which bounds the spectral norm, so the bound above holds with it;
* the score weighs the block's zero-order weight alpha_ij B (B = 64 tokens)
  by one plus that first-order discrepancy per token, with the router's
  pooled query qbar_i in place of q_t; ranking uses its logarithm
  s_ij + log1p(|qbar_i| M_j / (sqrt(d) B)), s_ij the plain logit (the
  constant log B is dropped).  Equal M_j for every block shift a row by a
  constant and leave the plain router's split unchanged; the split, counts
  and tie rule are those of ``oracle.sla``.

The evaluation subtracts the row max of all the exponents involved (exact
logits and centroid logits) from each of them, a common factor of N_t and
D_t.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from . import sla

BLOCK = sla.BLOCK


def block_statistics(k: np.ndarray, v: np.ndarray, block: int = BLOCK):
    """Per KV block: centroid kbar_j [nb, d], value sum [nb, d], token count n_j [nb],
    first-order matrix H_j = sum_n (k_n - kbar_j)^T v_n [nb, d, d].

    Pinned by: per-token brute force; H_j = 0 for constant key blocks.
    """
    n, d = k.shape
    nb = sla.n_blocks(n, block)
    kbar = np.empty((nb, d))
    vsum = np.empty((nb, v.shape[1]))
    cnt = np.empty(nb)
    H = np.empty((nb, d, v.shape[1]))
    for j, (a, b) in enumerate(sla.block_ranges(n, block)):
        kbar[j] = k[a:b].mean(axis=0)
        vsum[j] = v[a:b].sum(axis=0)
        cnt[j] = b - a
        H[j] = (k[a:b] - kbar[j]).T @ v[a:b]
    return kbar, vsum, cnt, H


def global_first_order(H: np.ndarray) -> np.ndarray:
    """Hbar: the mean of the per-block first-order matrices over all blocks."""
    return H.mean(axis=0)


def pisa_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, crit_idx: np.ndarray,
              block: int = BLOCK, q_blocks: Optional[Sequence[int]] = None):
    """o_t = N_t / D_t for one head; returns (o, o_softmax_part, o_correction_part).

    o_softmax_part = (exact + zero-order numerator) / D_t and
    o_correction_part = (first-order numerator) / D_t, so o is their sum.
    Rows outside ``q_blocks`` are 0.

    Pinned by: U_i empty gives dense softmax attention; constant key blocks
    make the expansion exact for any S_i; blocks with equal first-order
    matrices leave an error of second order in the key spread; per-token
    brute force on tiny inputs.
    """
    n, d = q.shape
    dv = v.shape[1]
    scale = 1.0 / math.sqrt(d)
    kbar, vsum, cnt, H = block_statistics(k, v, block)
    Hbar = global_first_order(H)
    ranges = sla.block_ranges(n, block)
    nb = len(ranges)
    o = np.zeros((n, dv))
    o_sm = np.zeros((n, dv))
    o_fo = np.zeros((n, dv))
    todo = range(nb) if q_blocks is None else q_blocks
    for i in todo:
        a, b = ranges[i]
        qs = q[a:b] * scale
        sel = np.asarray(crit_idx[i], dtype=np.int64)
        uns = np.setdiff1d(np.arange(nb), sel)
        toks = np.concatenate([np.arange(*ranges[j]) for j in sel]) if len(sel) else np.zeros(0, np.int64)
        x_ex = qs @ k[toks].T                      # exact logits   [rows, |tokens of S_i|]
        x_zo = qs @ kbar[uns].T                    # centroid logits [rows, |U_i|]
        m = np.full(b - a, -np.inf)
        if x_ex.size:
            m = np.maximum(m, x_ex.max(axis=1))
        if x_zo.size:
            m = np.maximum(m, x_zo.max(axis=1))
        e_ex = np.exp(x_ex - m[:, None])
        alpha = np.exp(x_zo - m[:, None])          # alpha_{t,j}, shifted by the row max
        num_sm = e_ex @ v[toks] + alpha @ vsum[uns]
        den = e_ex.sum(axis=1) + alpha @ cnt[uns]
        num_fo = (qs @ Hbar) * alpha.sum(axis=1, keepdims=True)
        o_sm[a:b] = num_sm / den[:, None]
        o_fo[a:b] = num_fo / den[:, None]
        o[a:b] = o_sm[a:b] + o_fo[a:b]
    return o, o_sm, o_fo


def block_deviation(H: np.ndarray, Hbar: np.ndarray) -> np.ndarray:
    """M_j = ||H_j - Hbar||, the L2 norm of the d x d deviation taken as a vector.

    Pinned by: squared norm = sum of squared singular values (numpy SVD);
    at least the spectral norm, so it bounds |q (H_j - Hbar)| / |q|; zero
    when every block shares one first-order matrix; brute-force loops.
    """
    dev = H - Hbar[None]
    return np.sqrt((dev * dev).sum(axis=(1, 2)))


def covariance_logits(q_pool: np.ndarray, k_pool: np.ndarray, M: np.ndarray,
                      block: int = BLOCK) -> np.ndarray:
    """s_ij + log1p(|qbar_i| M_j / (sqrt(d) B)), s_ij = qbar_i . kbar_j / sqrt(d).

    Pinned by: M = 0, or equal M_j for every block, gives the plain router's
    split; the logit grows with M_j and with nothing else of block j;
    brute-force loops.
    """
    d = q_pool.shape[1]
    s = (q_pool @ k_pool.T) / math.sqrt(d)
    c = np.sqrt((q_pool * q_pool).sum(axis=1)) / (math.sqrt(d) * block)
    return s + np.log1p(c[:, None] * M[None, :])


def route_pisa(q: np.ndarray, k: np.ndarray, v: np.ndarray, k_crit: int, k_marg: int,
               block: int = BLOCK):
    """Pool, covariance-aware score and split one head (outputs as ``sla.route``,
    plus the block deviations M_j and Hbar)."""
    qp = sla.pool(q, block)
    kp = sla.pool(k, block)
    _, _, _, H = block_statistics(k, v, block)
    Hbar = global_first_order(H)
    M = block_deviation(H, Hbar)
    logits = covariance_logits(qp, kp, M, block)
    crit, marg, cls = sla.select(logits, k_crit, k_marg)
    return {"crit_idx": crit, "marg_idx": marg, "block_class": cls, "logits": logits,
            "pooled_q": qp, "pooled_k": kp, "block_dev": M, "hbar": Hbar}
