"""OCP FP8 E4M3 ("e4m3fn") codec -- oracle side.  TEST INFRASTRUCTURE ONLY.

The preshuffled fp8 KV cache of "Beyond just running: native inference
optimisation in vLLM on AMD ROCm" (section "ROCM_AITER_FA", hardware-oriented KV
cache layout) stores one byte per element; the page does not name the fp8 flavour.
Reading taken: the OCP 8-bit floating point E4M3 format (the one gfx950 converts
natively), with a per-tensor scale, dequantised value = code * scale.

Format definition used here (OCP OFP8 E4M3):
  bit 7 sign, bits 6..3 exponent E (bias 7), bits 2..0 mantissa M.
  E == 0           : subnormal, value = M/8 * 2**-6
  1 <= E <= 15     : normal,    value = (1 + M/8) * 2**(E-7)
  E == 15, M == 7  : NaN (no infinities); largest finite = 1.75 * 2**8 = 448.

Encoding (the quantising cache write): round to the nearest representable
value, ties to the code with an even mantissa (round-half-to-even), magnitudes
beyond 448 saturate to 448, the sign is carried separately (so -0.0 -> 0x80).
This is implemented as a nearest-neighbour search over the 127 finite
non-negative code values -- deliberately not a bit-manipulation encoder.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0


def decode(codes: np.ndarray) -> np.ndarray:
    """fp8 e4m3fn codes (uint8) -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = (m / 8.0) * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


# The 127 finite non-negative values, indexed by their code 0x00..0x7E; they are
# strictly increasing in the code, so a sorted search finds the neighbours.
_POS_CODES = np.arange(0, 127, dtype=np.uint8)
_POS_VALUES = decode(_POS_CODES)
assert np.all(np.diff(_POS_VALUES) > 0)


def encode_rne_sat(y) -> np.ndarray:
    """float32 values -> e4m3fn codes, round-half-to-even, saturating at 448.

    NaN inputs map to 0x7F with their sign bit (never produced by the tests).
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)          # exact: float32 -> float64
    neg = np.signbit(y)
    hi = np.searchsorted(_POS_VALUES, a, side="left")   # first value >= a
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    v_hi = _POS_VALUES[hi]
    v_lo = _POS_VALUES[lo]
    d_hi = np.abs(v_hi - a)
    d_lo = np.abs(a - v_lo)
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    # ties: the code whose mantissa (low bit of the code) is even
    pick_hi = np.where(tie, (hi % 2) == 0, pick_hi)
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= MAX_FINITE, 126, code)          # saturate
    code = np.where(np.isnan(a), 127, code)
    code = code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)
    return code.astype(np.uint8)


def quantize(x_fp32, scale: float) -> np.ndarray:
    """The quantising store: code = encode(fl32(x) * fl32(1/scale)).

    Both the reciprocal and the product are single fp32 roundings, so the
    rounding decision is taken on exactly the same fp32 value on both sides of
    the parity test.
    """
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore"):
        y = np.asarray(x_fp32, dtype=np.float32) * inv   # overflow -> inf -> saturates
    return encode_rne_sat(y.astype(np.float32))
