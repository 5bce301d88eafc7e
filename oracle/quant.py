"""Per-token activation quantiser oracle (test infrastructure only).

Sources.  Humming: open-source kernel library for quantized inference
(news.ditty.ir), summary: W4A8 runs 4-bit weights against 8-bit activations
(INT8, or FP8 when the weights are MXFP4); cocoloop.cn (vi/fr), format
section: W4A8 and W4A8-MXFP4 are supported formats.  The pages do not say how
the 8-bit activations are produced.

Reading (the plainest symmetric per-row rule, listed with the others in the
design notes): for each row r of x,

    s[r]    = max_j |x[r, j]| / Q          (s[r] = 1 when the row is all zero)
    inv[r]  = 1 / s[r]
    code    = RNE(x[r, j] * inv[r])        saturated to [-Q, Q]

with Q = 448 and an OCP e4m3 ("fn") code for FP8, Q = 127 and a
two's-complement int8 code for INT8, so that code * s[r] approximates x.

The quotient is taken as a product with the row's reciprocal scale, the form
production per-token quantisers use (one multiply per element instead of a
division); code * s still approximates x within half a code step plus a few
float32 roundings.  A negative value that rounds to zero gives code 0 (no -0).

Precision.  The scale, its reciprocal and the product decide integer codes,
so the oracle takes them in IEEE float32, the precision the GPU kernel
computes in (numpy's float32 division and multiplication are correctly
rounded); the rounding of the float32 product to the code grid is then exact
(formats.rne / rint in float64 on a float32 value).  Inputs are fp16 / bf16
values, hence exact in float32.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_encode, e4m3_value, int8_value, ulp

Q_FP8 = 448.0
Q_INT8 = 127.0


def quantize_rows(x, out: str):
    """Quantise the rows of x (float array [m, k] of fp16/bf16 values).

    out "fp8" -> (uint8 e4m3 codes [m, k], float32 scales [m]);
    out "int8" -> (int8 codes [m, k], float32 scales [m]).
    """
    if out not in ("fp8", "int8"):
        raise ValueError("out must be 'fp8' or 'int8'")
    x32 = np.asarray(x, dtype=np.float32)
    if x32.ndim != 2:
        raise ValueError("x must be [m, k]")
    q = np.float32(Q_FP8 if out == "fp8" else Q_INT8)
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    s = np.where(amax > 0, amax / q, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)        # float32 reciprocal, correctly rounded
    v = (x32 * inv[:, None]).astype(np.float32)           # float32 product, correctly rounded
    v64 = np.clip(v.astype(np.float64), -float(q), float(q))
    if out == "fp8":
        return e4m3_encode(v64), s
    codes = np.clip(np.rint(v64), -127, 127).astype(np.int8)  # rint: ties to even
    return codes, s


def dequantize_rows(codes, scales, out: str) -> np.ndarray:
    """code value * s[r] in float64 (e4m3 or int8 codes)."""
    val = e4m3_value(np.asarray(codes)) if out == "fp8" else int8_value(np.asarray(codes))
    return val * np.asarray(scales, dtype=np.float64)[:, None]


def step_bound(x, scales, out: str) -> np.ndarray:
    """Half a code step at |x / s| times s: the rounding error bound of one
    element (plus 2^-22 relative for the float32 reciprocal and product)."""
    s = np.asarray(scales, dtype=np.float64)[:, None]
    v = np.abs(np.asarray(x, dtype=np.float64)) / s
    half = 0.5 * ulp(np.minimum(v, Q_FP8), "e4m3") if out == "fp8" else np.full_like(v, 0.5)
    return (half + 2.0 ** -22 * v) * s
