"""Plain fp64 reference of residual linear attention (test infrastructure only).

SPLA technical summary ("SPLA - Atención de Bloque Dispersa más Lineal para
el Modelado de Contexto Largo"):
* section 2.2: the blocks a query does not select are not dropped; their
  keys and values feed a linear-attention state, and the output of that
  branch is written as a difference, o_rla = o_bar - o_tilde, of linear
  attention over all blocks (o_bar) and over the selected blocks only
  (o_tilde), so the unselected blocks are never read one by one;
* section 2.3: the exact (sparse) branch and the residual branch are mixed
  by a gated sum, the residual output going through an RMS norm, and the
  feature map is a parameter-free exponential.

Readings fixed here where the page leaves a step open (each is listed in
the design notes):
* "linear attention" in the difference is the unnormalised form phi(q)^T S
  with S = sum of phi(k)^T v over the blocks concerned; the RMS norm that
  follows sets the scale, so no phi(q) . z denominator is taken;
* phi(k) = exp(k) elementwise, as is (no per-token normalisation); for the
  queries phi(q) = exp(q - max_a q_a), a per-row factor that the RMS norm
  removes (up to its epsilon);
* the RMS norm is over the d value features of each row, x / sqrt(mean(x^2)
  + eps) with eps = 1e-6 and unit scale (the trained scale parameters the
  page mentions are not available here);
* the gate is the per-head alpha of the SLA2 combination:
  O = alpha O_s + (1 - alpha) RMSNorm(o_rla);
* the selected blocks are the critical blocks of the router, so the
  residual state covers every non-critical block.

The sparse branch is the one of ``oracle.sla`` (exact softmax attention over
the critical blocks).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import sla

BLOCK = sla.BLOCK
RMS_EPS = 1e-6


def phi_exp(x: np.ndarray) -> np.ndarray:
    """Exponential feature map, elementwise (SPLA summary, section 2.3)."""
    return np.exp(x)


def linear_states_exp(k: np.ndarray, v: np.ndarray, block: int = BLOCK):
    """Per-block states with the exponential map: H_j = exp(K_j)^T V_j, z_j = colsum exp(K_j).

    Pinned by: brute force per token; a block whose keys share one row sum
    of exp(k) is that sum times the softmax-map state of ``oracle.sla``.
    """
    n, d = k.shape
    fk = phi_exp(k)
    nb = sla.n_blocks(n, block)
    H = np.empty((nb, d, v.shape[1]), dtype=np.float64)
    z = np.empty((nb, d), dtype=np.float64)
    for j, (a, b) in enumerate(sla.block_ranges(n, block)):
        H[j] = fk[a:b].T @ v[a:b]
        z[j] = fk[a:b].sum(axis=0)
    return H, z


def rla_branch(q: np.ndarray, H: np.ndarray, crit_idx: np.ndarray, block: int = BLOCK,
               q_blocks: Optional[Sequence[int]] = None) -> np.ndarray:
    """Unnormalised residual linear attention o_rla = o_bar - o_tilde per query block.

    o_bar[t] = phi(q_t) sum_j H_j over every block; o_tilde[t] = phi(q_t)
    sum_{j in C_i} H_j over the query block's critical blocks; phi(q_t) =
    exp(q_t - max q_t).  Taken literally as the difference of the two terms.
    Pinned by: per-token brute force over the non-critical tokens,
    sum_n (phi(q_t) . exp(k_n)) v_n.
    """
    n, d = q.shape
    out = np.zeros((n, H.shape[2]), dtype=np.float64)
    fq = np.exp(q - q.max(axis=1, keepdims=True))
    S_all = H.sum(axis=0)
    ranges = sla.block_ranges(n, block)
    todo = range(len(ranges)) if q_blocks is None else q_blocks
    for i in todo:
        a, b = ranges[i]
        o_bar = fq[a:b] @ S_all
        c = crit_idx[i]
        o_tilde = fq[a:b] @ H[c].sum(axis=0) if len(c) else np.zeros_like(o_bar)
        out[a:b] = o_bar - o_tilde
    return out


def rms_norm(x: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Each row divided by the root of (its mean square + eps), unit scale.

    Pinned by: rows of mean square 1 - eps come out unchanged; the output
    mean square is m / (m + eps) for input mean square m.
    """
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)


def forward_head_rla(q, k, v, crit_idx, H, alpha, block=BLOCK, q_blocks=None):
    """O = alpha O_s + (1 - alpha) RMSNorm(o_rla); returns (O, O_s, RMSNorm(o_rla)).

    Rows outside ``q_blocks`` are 0 in all three outputs.
    """
    o_s = sla.sparse_branch(q, k, v, crit_idx, block, q_blocks)
    o_r = rla_branch(q, H, crit_idx, block, q_blocks)
    if q_blocks is not None:
        rows = np.zeros(q.shape[0], dtype=bool)
        for i in set(q_blocks):
            a, b = sla.block_ranges(q.shape[0], block)[i]
            rows[a:b] = True
        o_n = np.zeros_like(o_r)
        o_n[rows] = rms_norm(o_r[rows])
    else:
        o_n = rms_norm(o_r)
    return sla.mix(o_s, o_n, alpha), o_s, o_n
