"""Exact decoding of the storage formats the path consumes (oracle, test infrastructure only).

bf16: the upper 16 bits of an IEEE-754 binary32; widening is exact.
e4m3fn (OCP 8-bit float, "FN" = finite + NaN, no infinities): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; largest finite 448.
The table below is built from that definition, not from any library.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """256-entry float64 table: code -> value of the OCP e4m3fn format."""
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if (code >> 7) & 1 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


_E4M3 = e4m3fn_table()


def decode_e4m3fn(u8: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> float64, exactly."""
    return _E4M3[np.asarray(u8, dtype=np.uint8)]


def dequant_rows(payload: np.ndarray, scale, dtype: str) -> np.ndarray:
    """Dequantise indexer rows to float64.

    bf16: exact widening (scale must be None).  fp8: code value times the fp32
    per-row scale (one scale per vector along the last axis); the product of an
    e4m3fn value and an fp32 is exact in float64.
    """
    if dtype == "bf16":
        assert scale is None
        return decode_bf16(payload)
    if dtype == "fp8":
        v = decode_e4m3fn(payload)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return v * s[..., None]
    raise ValueError(dtype)


def encode_e4m3fn(y) -> np.ndarray:
    """Finite float values with |y| <= 448 -> OCP e4m3fn codes, round to nearest, ties
    to the even mantissa; the sign is kept (-0.0 and negatives that round to zero give
    0x80).  Written from the format definition: the nearest of the 127 finite
    non-negative magnitudes (codes 0x00 .. 0x7E), by exhaustive comparison."""
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y)) and np.all(np.abs(y) <= 448.0)
    mags = _E4M3[:0x7F]                       # increasing in the code
    a = np.abs(y)[..., None]
    d = np.abs(a - mags)                      # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                          # one code, or two at a tie
    codes = np.arange(0x7F)
    even = (codes & 1) == 0
    pick = np.where(cand & even, codes, 0x7F).min(axis=-1)        # tie: the even mantissa
    single = np.where(cand, codes, 0x7F).min(axis=-1)
    code = np.where(cand.sum(axis=-1) > 1, pick, single).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def quantize_fp8_rows(x: np.ndarray):
    """Per-row quantisation of the indexer inputs, in fp32 arithmetic (the precision
    that takes the rounding decision): scale = amax/448 over the row (1 for an all-zero
    row), y = clamp(x / scale, +-448), codes = encode_e4m3fn(y).  Returns (codes uint8,
    scales float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[..., None], np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    return encode_e4m3fn(y), scale
