"""Shared helpers for the GPU parity tests: mask comparison with the tie
rule, error metrics, and tensor conversions (no method arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

TIE_WINDOW = 1e-5      # |logit difference| that excuses a boundary disagreement
REL_L2_BF16 = 1e-2
MAX_ABS_BF16 = 2e-2
REL_L2_FP8 = 5e-2       # fp8 sparse branch against the unquantised oracle:
MAX_ABS_FP8 = 5e-2      # both metrics take the 5e-2 bound


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (nb if nb > 0 else 1.0))


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def check_index_lists(crit: np.ndarray, marg: np.ndarray, nkb: int):
    """Structural validity of one head's lists: ascending, in range, disjoint."""
    for i in range(crit.shape[0]):
        c, m = crit[i], marg[i]
        assert (np.diff(c) > 0).all() and (np.diff(m) > 0).all(), f"row {i} not ascending"
        assert c.size == 0 or (c.min() >= 0 and c.max() < nkb)
        assert m.size == 0 or (m.min() >= 0 and m.max() < nkb)
        assert len(np.intersect1d(c, m)) == 0, f"row {i}: critical and marginal overlap"


def classes_from_lists(crit: np.ndarray, marg: np.ndarray, nkb: int) -> np.ndarray:
    cls = np.zeros((crit.shape[0], nkb), dtype=np.int8)
    rows = np.arange(crit.shape[0])[:, None]
    if marg.shape[1]:
        cls[rows, marg] = 1
    if crit.shape[1]:
        cls[rows, crit] = 2
    return cls


def compare_classes(gpu_cls: np.ndarray, ora_cls: np.ndarray, logits: np.ndarray, kc: int, km: int):
    """Count disagreements; excused iff the block's oracle logit lies within
    TIE_WINDOW of the oracle's boundary logit(s) it crosses.  Returns
    (excused, unexcused, rows_with_excused)."""
    excused = unexcused = 0
    rows = set()
    srt = -np.sort(-logits, axis=1)
    bad_i, bad_j = np.nonzero(gpu_cls != ora_cls)
    for i, j in zip(bad_i, bad_j):
        a, b = int(gpu_cls[i, j]), int(ora_cls[i, j])
        ranks = []
        if max(a, b) == 2 and min(a, b) <= 1:
            ranks.append(kc)
        if min(a, b) == 0 and max(a, b) >= 1:
            ranks.append(kc + km)
        ok = all(abs(logits[i, j] - srt[i, r - 1]) <= TIE_WINDOW or
                 (r < srt.shape[1] and abs(logits[i, j] - srt[i, r]) <= TIE_WINDOW)
                 for r in ranks)
        if ok:
            excused += 1
            rows.add(int(i))
        else:
            unexcused += 1
    return excused, unexcused, len(rows)


def metrics_by_head(pairs):
    """pairs: {head label: (got, ref)} float64 arrays of one output.
    Returns (whole-tensor (rel L2, max-abs), {label: (rel L2, max-abs)})."""
    per = {lab: (rel_l2(a, b), max_abs(a, b)) for lab, (a, b) in pairs.items()}
    got = np.concatenate([a.ravel() for a, _ in pairs.values()])
    ref = np.concatenate([b.ravel() for _, b in pairs.values()])
    return (rel_l2(got, ref), max_abs(got, ref)), per


def format_per_head(per) -> str:
    return " ".join(f"{lab}:{e:.1e}/{m:.1e}" for lab, (e, m) in per.items())
