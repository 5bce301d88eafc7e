"""Number formats, nibble unpacking and exact rounding (oracle; test infrastructure).

Everything here is written from the definition of each format and checked in
tests/test_oracle.py against tables derived independently (hand-written
literals, torch's fp8 decoders, numpy's float16 cast).

Readings (the pages name the formats -- INT4, MXFP4, FP8 -- but define none):

* Canonical INT4 / E2M1 packing: 8 codes per 32-bit word along K, code k = 8j+i
  in bits [4i, 4i+4) of word j (low nibble first).  The 32-bit word is only a
  bit container; its sign is irrelevant, so unpacking uses unsigned shifts.
* E2M1 (OCP MX v1.0, FP4 element type): sign, 2 exponent bits (bias 1),
  1 mantissa bit; exponent field 0 is subnormal (value m/2).  No inf/NaN.
* E8M0 (OCP MX v1.0, shared scale): 2^(X-127); X = 255 is NaN.
* E4M3 (OCP 8-bit FP, "fn" variant): sign, 4 exponent bits (bias 7),
  3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is
  NaN; there is no infinity; the largest finite magnitude is 448.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# nibble unpack (canonical layout)
# --------------------------------------------------------------------------


def unpack_u4(words) -> np.ndarray:
    """Unpack int32 words [..., K/8] into uint8 codes [..., K], low nibble first.

    Code k = 8*j + i is bits [4i, 4i+4) of word j.  The words are reinterpreted
    as uint32 so that a word with bit 31 set unpacks the same as any other.
    """
    w = np.ascontiguousarray(words).view(np.uint32)
    out = np.empty(w.shape[:-1] + (w.shape[-1] * 8,), dtype=np.uint8)
    for i in range(8):
        out[..., i::8] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    return out


# --------------------------------------------------------------------------
# code -> value, straight from each format's definition
# --------------------------------------------------------------------------


def e2m1_value(code) -> np.ndarray:
    """OCP MX E2M1 element value of a 4-bit code (array of ints in [0, 16))."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    normal = np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64))
    sub = m / 2.0  # exponent field 0: 2^(1-bias) * (m/2) with bias 1
    return sign * np.where(e == 0, sub, normal)


def mxint4_value(code) -> np.ndarray:
    """MXINT4 element value of a 4-bit code: the code read as a two's-complement
    integer (-8..7) times an implicit 2^-2, i.e. a 1.2 fixed-point number in
    [-2, 1.75] -- the 4-bit form of the OCP MX integer element, whose 8-bit
    form (MXINT8) is a two's-complement integer times 2^-6."""
    c = np.asarray(code, dtype=np.int64)
    return np.where(c >= 8, c - 16, c) * 0.25


def e8m0_value(code) -> np.ndarray:
    """OCP MX E8M0 shared-scale value 2^(X-127); X = 255 decodes to NaN."""
    x = np.asarray(code, dtype=np.int64)
    v = np.ldexp(1.0, (x - 127).astype(np.int64))
    return np.where(x == 255, np.nan, v)


def e4m3_value(code) -> np.ndarray:
    """OCP FP8 E4M3 ("fn": no inf, NaN = S.1111.111) value of an 8-bit code."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def int8_value(code) -> np.ndarray:
    """Two's-complement int8 code -> value (codes given as uint8 or int8)."""
    c = np.asarray(code).astype(np.int64)
    return np.where(c >= 128, c - 256, c).astype(np.float64)


# --------------------------------------------------------------------------
# exact round-to-nearest-even from float64
# --------------------------------------------------------------------------

# (significant bits p, smallest normal exponent emin)
_FMT = {
    "f16": (11, -14),
    "bf16": (8, -126),
    "e4m3": (4, -6),
    "e2m1": (2, 0),
    "f32": (24, -126),
}


def rne(x, fmt: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``fmt`` (ties to even).

    A value with binary exponent e (2^e <= |x| < 2^(e+1)) is rounded on the
    grid 2^(max(e, emin) - p + 1); below the smallest normal the grid is the
    subnormal spacing.  The division by a power of two and ``np.rint`` (ties
    to even) are exact in float64, so the only rounding is the intended one.
    Overflow is not handled: callers keep values inside the finite range.
    """
    p, emin = _FMT[fmt]
    x = np.asarray(x, dtype=np.float64)
    _, E = np.frexp(np.abs(x))  # |x| = f * 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, emin)
    ulp = np.ldexp(1.0, e - (p - 1))
    return np.rint(x / ulp) * ulp


def ulp(x, fmt: str) -> np.ndarray:
    """Spacing of ``fmt`` values at magnitude |x| (the grid ``rne`` rounds on)."""
    p, emin = _FMT[fmt]
    _, E = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    e = np.maximum(E - 1, emin)
    return np.ldexp(1.0, e - (p - 1))


def e2m1_encode(x) -> np.ndarray:
    """Code of RNE_e2m1(x) for finite |x| <= 6 (callers clamp first); a value
    that rounds to zero gives code 0 (no -0)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > 6.0) or np.any(np.isnan(x)):
        raise ValueError("e2m1_encode expects finite values with |x| <= 6")
    r = rne(x, "e2m1")
    pos = e2m1_value(np.arange(8))  # 0, 0.5, 1, 1.5, 2, 3, 4, 6: increasing
    idx = np.searchsorted(pos, np.abs(r))
    if not np.all(pos[np.minimum(idx, 7)] == np.abs(r)):
        raise AssertionError("rounded value is not an e2m1 value")
    code = idx.astype(np.int64)
    code = np.where(np.signbit(r) & (r != 0), code | 0x8, code)
    return code.astype(np.uint8)


def e4m3_encode(x) -> np.ndarray:
    """Code of RNE_e4m3(x) for finite |x| <= 448 (callers clamp first)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > 448.0) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode expects finite values with |x| <= 448")
    r = rne(x, "e4m3")
    table = e4m3_value(np.arange(256))
    # positive codes 0..126 are strictly increasing in value
    pos = table[:127]
    idx = np.searchsorted(pos, np.abs(r))
    if not np.all(pos[np.minimum(idx, 126)] == np.abs(r)):
        raise AssertionError("rounded value is not an e4m3 value")
    code = idx.astype(np.int64)
    code = np.where(np.signbit(r) & (r != 0), code | 0x80, code)
    return code.astype(np.uint8)
