"""Pins for the oracle's fp8 e4m3fn codec (CPU only).

What fixes the codec independently of the oracle's own code:
* the OCP E4M3 format definition: a handful of anchor codes;
* torch's float8_e4m3fn conversion (a library routine the oracle does not
  use), exhaustively over every finite bf16 pattern at several scales;
* the round-half-to-even rule at explicit midpoints, and saturation.
"""
import math

import numpy as np
import pytest

from oracle import fp8


def test_decode_anchor_codes():
    # sign | exponent (bias 7) | mantissa, per the OCP E4M3 definition
    anchors = {
        0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x3C: 1.5,
        0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
        0x07: 7 * 2.0 ** -9, 0x77: 240.0, 0x78: 256.0,
    }
    for c, v in anchors.items():
        assert fp8.decode(np.uint8(c)) == v, hex(c)
    assert math.isnan(fp8.decode(np.uint8(0x7F)))
    assert math.isnan(fp8.decode(np.uint8(0xFF)))
    assert np.signbit(fp8.decode(np.uint8(0x80)))


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.decode(codes).astype(np.float32)
    back = fp8.encode_rne_sat(vals)
    assert np.array_equal(back, codes)


def test_midpoints_round_to_even_and_saturate():
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39)
    assert fp8.encode_rne_sat(np.float32(1.0625)) == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even)
    assert fp8.encode_rne_sat(np.float32(1.1875)) == 0x3A
    # halfway between the two smallest subnormals 2^-9 (0x01) and 2^-8 (0x02)
    assert fp8.encode_rne_sat(np.float32(1.5 * 2.0 ** -9)) == 0x02
    # below half the smallest subnormal -> zero; exactly half -> zero (even)
    assert fp8.encode_rne_sat(np.float32(2.0 ** -10)) == 0x00
    assert fp8.encode_rne_sat(np.float32(-(2.0 ** -10))) == 0x80
    # saturation instead of NaN
    for big in (448.0, 460.0, 464.0, 1e4, 3.0e38):
        assert fp8.encode_rne_sat(np.float32(big)) == 0x7E
        assert fp8.encode_rne_sat(np.float32(-big)) == 0xFE


@pytest.mark.parametrize("scale", [1.0, 0.0136, 1.0 / 64, 0.37, 3.0])
def test_against_torch_cast_all_bf16(scale):
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x)]
    ours = fp8.quantize(x, scale)
    with np.errstate(over="ignore"):
        y = x * (np.float32(1.0) / np.float32(scale))
    inrange = np.abs(y) < 464.0          # torch rounds up to 448 below 464, NaN above
    ref = torch.from_numpy(y[inrange]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours[inrange], ref)
    big = ~inrange
    assert np.all(ours[big & (y > 0)] == 0x7E)
    assert np.all(ours[big & (y < 0)] == 0xFE)
