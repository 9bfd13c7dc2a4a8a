"""Emulation of the low-bit sparse branch's number format (test infrastructure only).

The SLA2 technical summary (section 2.C) runs the sparse branch in a low-bit
format ("INT8/FP8") with quantisation-aware training.  The reading taken here
is the OCP 8-bit floating-point E4M3 format that gfx950's matrix cores use:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* no infinities; exponent 1111 with mantissa 111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448;
* subnormals m * 2^-9, m = 1..7; the smallest normal is 2^-6.

Conversion from float32 rounds to nearest, ties to even, and saturates
finite values beyond 448 to +-448.  The quantiser scales each 64-token block
of a head by its absolute maximum:

    r = fl32(448 / absmax),  scale = fl32(absmax / 448),
    code = e4m3(fl32(x * r))

and a block whose absmax is 0 gets scale 1 (its codes are all +0).
Every step is float32 arithmetic, emulated here with numpy float32 ops, so
the GPU quantiser must match these bytes exactly.

Pinned by: the encoder equals torch's float8_e4m3fn CPU cast (after the
saturation clamp) on every bfloat16 value and on random float32 values;
spec values (448 -> 0x7E, 2^-9 -> 0x01, 2^-10 -> 0x00, ...); decode(encode)
round-trips every finite code.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_BIAS = 7


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** (1 - _BIAS - 3),
                   (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - _BIAS))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def encode_e4m3(x) -> np.ndarray:
    """float32 values -> uint8 E4M3 codes, round-to-nearest-even, saturating.

    Works in float64, where every step below is exact for float32 inputs:
    the magnitude is divided by its quantum (a power of two), rounded with
    numpy's half-to-even ``rint``, and the code assembled from the result.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no saturating E4M3 encoding here")
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    # exponent of the binade (frexp is exact), clamped to the subnormal
    # binade (-6 is the smallest normal exponent; below it the quantum stays 2^-9)
    e = np.frexp(np.where(a > 0, a, 1.0))[1].astype(np.float64) - 1.0
    e = np.clip(e, -6, 8)
    quantum = np.exp2(e - 3)
    q = np.rint(a / quantum) * quantum          # RNE to the binade's grid
    q = np.minimum(q, E4M3_MAX)                 # saturate (incl. rounding past 448)
    # assemble the code from the rounded magnitude
    qe = np.frexp(np.where(q > 0, q, 1.0))[1].astype(np.float64) - 1.0
    normal = q >= 2.0 ** -6
    exp_field = np.where(normal, qe + _BIAS, 0).astype(np.int64)
    mant = np.where(normal, np.rint((q / np.exp2(qe) - 1.0) * 8.0),
                    np.rint(q / 2.0 ** -9)).astype(np.int64)
    mant = np.where(q == 0, 0, mant)
    exp_field = np.where(q == 0, 0, exp_field)
    code = (exp_field << 3) | mant
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_blocks(x: np.ndarray, block: int = 64):
    """Per-block E4M3 quantisation of one head's rows.

    ``x``: [N, d] float32 values (what the GPU sees after upcasting its
    input).  Returns (codes uint8 [N, d], scales float32 [nb]).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    nb = (n + block - 1) // block
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.ones(nb, dtype=np.float32)
    for j in range(nb):
        a, b = j * block, min((j + 1) * block, n)
        blk = x[a:b]
        amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
        if amax == 0:
            scales[j] = np.float32(1.0)
            codes[a:b] = encode_e4m3(blk)
            continue
        r = np.float32(E4M3_MAX) / amax
        scales[j] = amax / np.float32(E4M3_MAX)
        codes[a:b] = encode_e4m3((blk * r).astype(np.float32))
    return codes, scales


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 64) -> np.ndarray:
    """Values the codes stand for: decode(code) * the scale of the row's block.

    Pinned by: hand-derived values for codes the format fixes under
    different block scales (a short last block included); the round trip
    through ``quantize_blocks`` stays within half a quantum of the scaled
    E4M3 grid.
    """
    n = codes.shape[0]
    out = decode_e4m3(codes)
    for j in range(len(scales)):
        a, b = j * block, min((j + 1) * block, n)
        out[a:b] *= float(scales[j])
    return out


def quantize_blocks_batched(x: np.ndarray, block: int = 64):
    B, H = x.shape[:2]
    codes = np.zeros(x.shape, dtype=np.uint8)
    nb = (x.shape[2] + block - 1) // block
    scales = np.zeros((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            codes[b, h], scales[b, h] = quantize_blocks(x[b, h], block)
    return codes, scales
