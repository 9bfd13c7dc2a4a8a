"""Pins of the E4M3 emulation in the oracle (CPU only).

The encoder is checked against torch's float8_e4m3fn CPU conversion (a
library routine; torch turns out-of-range values into NaN, so inputs are
clamped to the saturation bound first), against values fixed by the OCP
8-bit floating-point format, and by round trips over every code.
"""
import numpy as np
import pytest
import torch

from oracle import fp8


def _all_bf16_as_f32():
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    return bits[np.isfinite(bits)]


@pytest.mark.parametrize("scale", [1.0, 448.0 / 3.0, 2.0 ** -7, 1000.0, 0.3])
def test_encoder_matches_torch_on_every_bf16_value(scale):
    with np.errstate(over="ignore"):
        x = (_all_bf16_as_f32() * np.float32(scale)).astype(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8.encode_e4m3(x), ref)


def test_encoder_matches_torch_on_random_f32():
    r = np.random.default_rng(3)
    x = (r.standard_normal(200000) * np.exp2(r.integers(-14, 10, 200000))).astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8.encode_e4m3(x), ref)


def test_spec_values():
    x = np.array([448, 464, 480, 1e9, 2 ** -6, 2 ** -9, 2 ** -10, 1.5 * 2 ** -10, 1.0, 1.0625, 1.1875,
                  -0.0, -448, 3 * 2 ** -9], dtype=np.float32)
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x08, 0x01, 0x00, 0x01, 0x38, 0x38, 0x3A, 0x80, 0xFE, 0x03]
    np.testing.assert_array_equal(fp8.encode_e4m3(x), want)
    np.testing.assert_array_equal(fp8.decode_e4m3(np.array([0x7E, 0x08, 0x01, 0x38, 0xFE], dtype=np.uint8)),
                                  [448.0, 2 ** -6, 2 ** -9, 1.0, -448.0])
    assert np.isnan(fp8.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_round_trip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.decode_e4m3(codes).astype(np.float32)
    np.testing.assert_array_equal(fp8.encode_e4m3(vals), codes)


def test_block_quantiser_properties():
    r = np.random.default_rng(5)
    x = r.standard_normal((64 * 3 + 10, 32)).astype(np.float32)
    x[64:128] = 0.0
    codes, scales = fp8.quantize_blocks(x)
    assert scales[1] == 1.0 and (codes[64:128] == 0).all()
    for j, (a, b) in enumerate([(0, 64), (128, 192), (192, 202)]):
        jj = [0, 2, 3][j]
        amax = np.abs(x[a:b]).max()
        assert scales[jj] == np.float32(amax / np.float32(448.0))
        # the block's largest magnitude lands on the top code
        assert (np.abs(fp8.decode_e4m3(codes[a:b])).max()) == 448.0
        deq = fp8.decode_e4m3(codes[a:b]) * scales[jj]
        big = np.abs(x[a:b]) >= amax * 2.0 ** -6      # normal range: relative error <= 2^-4
        assert (np.abs(deq - x[a:b])[big] <= np.abs(x[a:b])[big] * 2.0 ** -4 + 1e-12).all()


def test_dequantize_blocks_hand_values():
    # two blocks of 64 rows and a 3-row tail; codes with values fixed by the
    # format: 0x38 = 1, 0x7E = 448, 0x01 = 2^-9, 0xC0 = -2, 0x00 = 0,
    # 0x3C = 1.5; each row is multiplied by its own block's scale
    codes = np.zeros((131, 2), dtype=np.uint8)
    codes[0] = [0x38, 0x7E]
    codes[63] = [0x01, 0xC0]
    codes[64] = [0x38, 0x3C]
    codes[130] = [0x7E, 0xC0]
    scales = np.array([2.0, 0.25, 1.0 / 448.0], dtype=np.float32)
    out = fp8.dequantize_blocks(codes, scales)
    want = np.zeros((131, 2))
    want[0] = [2.0, 896.0]
    want[63] = [2.0 ** -8, -4.0]
    want[64] = [0.25, 0.375]
    want[130] = [float(np.float32(1.0 / 448.0)) * 448.0, -2.0 * float(np.float32(1.0 / 448.0))]
    np.testing.assert_array_equal(out, want)


def test_dequantize_inverts_quantize_within_the_format_error():
    # x -> codes, scale -> x': each element is within half a quantum of the
    # block-scaled grid: relative 2^-4 in the normal range, and at most
    # 2^-10 * scale (half the subnormal step) below it
    r = np.random.default_rng(11)
    x = (r.standard_normal((64 * 5 + 9, 128)) * np.exp2(r.integers(-6, 6, (64 * 5 + 9, 1)))).astype(np.float32)
    codes, scales = fp8.quantize_blocks(x)
    deq = fp8.dequantize_blocks(codes, scales)
    for j in range(len(scales)):
        a, b = 64 * j, min(64 * j + 64, x.shape[0])
        err = np.abs(deq[a:b] - x[a:b])
        bound = np.maximum(np.abs(x[a:b]) * 2.0 ** -4, 2.0 ** -10 * float(scales[j])) * (1 + 1e-6)
        assert (err <= bound).all(), j
        # the block's largest magnitude is reproduced to float32 rounding
        amax = np.abs(x[a:b]).max()
        assert abs(np.abs(deq[a:b]).max() - amax) <= amax * 2.0 ** -20
