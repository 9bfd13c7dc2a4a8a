"""Seeded synthetic inputs shaped like the pages' video-DiT attention workloads.

The pages (SLA2 and SALAD technical summaries, results sections; the SLA
abstract) measure on Wan2.1 video diffusion transformers at 30k-100k tokens.
Those activations are not available, so tensors are synthesised here:

* positions on a token raster (1-D index, or a (t, y, x) latent grid in
  row-major order with x fastest);
* Q and K share one smooth random-Fourier-feature field of the position,
  projected to the head dimension, plus independent Gaussian noise, so that
  Q.K^T favours nearby tokens the way video attention maps do;
* V is i.i.d. N(0, 1);
* the per-head mixing weight alpha is drawn from U(0.3, 0.9).

Every array is drawn in float64 from ``numpy.random.Generator(PCG64(seed))``
and cast once to the workload dtype (float64 -> float32 -> bfloat16, each
step round-to-nearest-even).  Layout is ``[B, H, N, d]`` contiguous.

Draw order per head: Fourier frequencies, phases, projection W, then the Q
noise, the K noise and V.  The alpha vector is drawn last.  Nothing in this
module computes any part of the attention method.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

BLOCK = 64


def num_blocks(n: int, block: int = BLOCK) -> int:
    """Number of blocks of ``block`` consecutive tokens covering ``n`` tokens."""
    return (n + block - 1) // block


def band_count(frac: float, nkb: int) -> int:
    """Round a density band (e.g. 'top 5 %') to a block count: floor(frac*nkb + 1/2)."""
    return int(math.floor(frac * nkb + 0.5))


@dataclasses.dataclass
class Workload:
    name: str
    q: torch.Tensor          # [B, H, N, d] in the workload dtype (CPU)
    k: torch.Tensor
    v: torch.Tensor
    alpha: torch.Tensor      # [H] float32
    k_crit: int
    k_marg: int
    meta: dict

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return tuple(self.q.shape)  # type: ignore[return-value]


# name -> (B, H, N, d, dtype, positional kind, grid, n_freq, length scales,
#          critical fraction / explicit count, marginal fraction / count)
CONFIGS = {
    # tiny CPU-checkable case: fp32 i.i.d. normal, 16 blocks, 4/8/4 split
    "tiny": dict(B=1, H=2, N=1024, d=64, dtype="fp32", kind="iid",
                 k_crit=4, k_marg=8, alpha=(0.6, 0.4), seed=1001),
    # 1-D sequence, 16 Fourier frequencies, 10 % / 20 % bands
    "seq8k": dict(B=1, H=12, N=8192, d=128, dtype="bf16", kind="fourier1d",
                  n_freq=16, ell=256.0, p_crit=0.10, p_marg=0.20, seed=1002),
    # video-DiT latent 21 x 30 x 52, 32 frequencies, 5 % / 10 % bands
    "video32k": dict(B=1, H=12, N=32760, d=128, dtype="bf16", kind="fourier3d",
                     grid=(21, 30, 52), n_freq=32, ell=(3.0, 6.0, 6.0),
                     p_crit=0.05, p_marg=0.10, seed=1003),
    # larger video-DiT latent 21 x 45 x 80, 40 heads
    "video75k": dict(B=1, H=40, N=75600, d=128, dtype="bf16", kind="fourier3d",
                     grid=(21, 45, 80), n_freq=32, ell=(3.0, 6.0, 6.0),
                     p_crit=0.05, p_marg=0.10, seed=1004),
    # the 32k video shape with the fp8 sparse branch (same tensors as video32k)
    "video32k_fp8": dict(B=1, H=12, N=32760, d=128, dtype="bf16", kind="fourier3d",
                         grid=(21, 30, 52), n_freq=32, ell=(3.0, 6.0, 6.0),
                         p_crit=0.05, p_marg=0.10, seed=1003, fp8=True),
}


def _cast(x64: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x64.astype(np.float32)))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    return t


def _positions(kind: str, n: int, grid) -> np.ndarray:
    if kind == "fourier1d":
        return np.arange(n, dtype=np.float64)[:, None]
    t, y, x = grid
    assert t * y * x == n
    tt, yy, xx = np.meshgrid(np.arange(t), np.arange(y), np.arange(x), indexing="ij")
    return np.stack([tt.ravel(), yy.ravel(), xx.ravel()], axis=1).astype(np.float64)


def _head_qkv(rng: np.random.Generator, pos: np.ndarray, d: int, n_freq: int,
              ell) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    dim = pos.shape[1]
    ell = np.broadcast_to(np.asarray(ell, dtype=np.float64), (dim,))
    omega = rng.standard_normal((n_freq, dim)) / ell[None, :]
    beta = rng.uniform(0.0, 2.0 * np.pi, size=n_freq)
    w = rng.standard_normal((2 * n_freq, d)) / math.sqrt(n_freq)
    ang = pos @ omega.T + beta[None, :]
    feat = np.concatenate([np.cos(ang), np.sin(ang)], axis=1) @ w
    n = pos.shape[0]
    eq = rng.standard_normal((n, d))
    ek = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    return 0.7 * feat + 0.3 * eq, 0.7 * feat + 0.3 * ek, v


def make_custom(B: int, H: int, N: int, d: int, dtype: str = "bf16", kind: str = "fourier1d",
                seed: int = 0, k_crit: Optional[int] = None, k_marg: Optional[int] = None,
                p_crit: float = 0.1, p_marg: float = 0.2, grid=None, n_freq: int = 16,
                ell=None, alpha=None, name: str = "custom") -> Workload:
    """Build a workload of any shape with the same recipe as the named ones."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nkb = num_blocks(N)
    if k_crit is None:
        k_crit = band_count(p_crit, nkb)
    if k_marg is None:
        k_marg = band_count(p_marg, nkb)
    k_marg = max(0, min(k_marg, nkb - k_crit))
    if kind == "iid":
        q = rng.standard_normal((B, H, N, d))
        k = rng.standard_normal((B, H, N, d))
        v = rng.standard_normal((B, H, N, d))
    else:
        if ell is None:
            ell = 256.0 if kind == "fourier1d" else (3.0, 6.0, 6.0)
        pos = _positions(kind, N, grid)
        q = np.empty((B, H, N, d))
        k = np.empty((B, H, N, d))
        v = np.empty((B, H, N, d))
        for b in range(B):
            for h in range(H):
                q[b, h], k[b, h], v[b, h] = _head_qkv(rng, pos, d, n_freq, ell)
    if alpha is None:
        alpha = rng.uniform(0.3, 0.9, size=H)
    alpha = torch.tensor(np.asarray(alpha, dtype=np.float64), dtype=torch.float32)
    meta = dict(B=B, H=H, N=N, d=d, dtype=dtype, kind=kind, seed=seed, nkb=nkb,
                k_crit=k_crit, k_marg=k_marg, grid=grid, n_freq=n_freq,
                ell=ell if ell is None or np.isscalar(ell) else list(ell))
    return Workload(name, _cast(q, dtype), _cast(k, dtype), _cast(v, dtype), alpha,
                    k_crit, k_marg, meta)


def _make_named_uncached(name: str) -> Workload:
    c = CONFIGS[name]
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    nkb = num_blocks(N)
    if c["kind"] == "iid":
        return make_custom(B, H, N, d, dtype=c["dtype"], kind="iid", seed=c["seed"],
                           k_crit=c["k_crit"], k_marg=c["k_marg"], alpha=c["alpha"],
                           name=name)
    kc = band_count(c["p_crit"], nkb)
    km = band_count(c["p_marg"], nkb)
    return make_custom(B, H, N, d, dtype=c["dtype"], kind=c["kind"], seed=c["seed"],
                       k_crit=kc, k_marg=km, grid=c.get("grid"), n_freq=c["n_freq"],
                       ell=c["ell"], name=name)


_CACHE: dict = {}


def make_workload(name: str, cache: bool = True) -> Workload:
    """Return the named workload (deterministic; cached per process)."""
    if cache and name in _CACHE:
        return _CACHE[name]
    w = _make_named_uncached(name)
    if cache:
        _CACHE[name] = w
    return w
