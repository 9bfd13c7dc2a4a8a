"""Plain fp64 reference of the second-order block routing score (test infrastructure only).

SPLA technical summary ("SPLA - Atención de Bloque Dispersa más Lineal para
el Modelado de Contexto Largo"), section 2.1: a block's relevance is the
attention mass of all its tokens; expanding the exponential score around the
block mean to second order gives exp(q^T kbar) (1 + 1/2 q^T Cov(k) q), with
the covariance taken diagonal so that only per-feature block variances are
kept.

Readings fixed here (each is listed in the design notes):
* the query is the pooled query block qbar_i, as for the SLA router, and the
  score keeps the standard 1/sqrt(d) scaling: q' = qbar_i / sqrt(d);
* Cov(k) is the population covariance of the block's valid keys (divided by
  n_j), diagonal part only: var_ja = mean_n (k_na - kbar_ja)^2;
* ranking uses the logarithm of the score,
  s_ij = qbar_i . kbar_j / sqrt(d) + log1p(sum_a qbar_ia^2 var_ja / (2 d)),
  a monotone transform; the split into critical / marginal / negligible and
  the tie rule (lower block index first) are those of ``oracle.sla``.
"""
from __future__ import annotations

import math

import numpy as np

from . import sla

BLOCK = sla.BLOCK


def block_variance(x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Per-block population variance of each feature: [N, d] -> [nb, d].

    Pinned by: constant blocks give 0; one feature set to +-c alternately in
    a block of even length gives c^2.
    """
    n, d = x.shape
    out = np.empty((sla.n_blocks(n, block), d), dtype=np.float64)
    for j, (a, b) in enumerate(sla.block_ranges(n, block)):
        m = x[a:b].mean(axis=0)
        out[j] = ((x[a:b] - m) ** 2).mean(axis=0)
    return out


def taylor_logits(q_pool: np.ndarray, k_pool: np.ndarray, k_var: np.ndarray) -> np.ndarray:
    """s_ij = qbar_i . kbar_j / sqrt(d) + log1p(sum_a qbar_ia^2 var_ja / (2 d)).

    Pinned by: zero variance gives the SLA logits; the score approaches the
    block mean of exp(q' . k) as the spread shrinks (error of third order).
    """
    d = q_pool.shape[1]
    first = (q_pool @ k_pool.T) / math.sqrt(d)
    second = ((q_pool * q_pool) @ k_var.T) / (2.0 * d)
    return first + np.log1p(second)


def route_taylor(q: np.ndarray, k: np.ndarray, k_crit: int, k_marg: int, block: int = BLOCK):
    """Pool, second-order score and split one head (same outputs as ``sla.route``)."""
    qp = sla.pool(q, block)
    kp = sla.pool(k, block)
    kv = block_variance(k, block)
    logits = taylor_logits(qp, kp, kv)
    crit, marg, cls = sla.select(logits, k_crit, k_marg)
    return {"crit_idx": crit, "marg_idx": marg, "block_class": cls, "logits": logits,
            "pooled_q": qp, "pooled_k": kp, "k_var": kv}
