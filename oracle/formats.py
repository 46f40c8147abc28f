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
