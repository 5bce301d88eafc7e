"""Per-token activation quantiser oracle (test infrastructure only).

Sources.  Humming: open-source kernel library for quantized inference
(news.ditty.ir), summary: W4A8 runs 4-bit weights against 8-bit activations
(INT8, or FP8 when the weights are MXFP4); cocoloop.cn (vi/fr), format
section: W4A8 and W4A8-MXFP4 are supported formats.  The pages do not say how
the 8-bit activations are produced.

Reading (the plainest symmetric per-row rule, listed with the others in the
design notes): for each row r of x,

    s[r]    = max_j |x[r, j]| / Q          (s[r] = 1 when the row is all zero)
    code    = RNE(x[r, j] / s[r])          saturated to [-Q, Q]

with Q = 448 and an OCP e4m3 ("fn") code for FP8, Q = 127 and a
two's-complement int8 code for INT8, so that code * s[r] approximates x.  The
quotient is the correctly rounded float32 division (one rounding), the same
rule the fused requantisation of the MoE gate_up output follows.  A negative
value that rounds to zero gives code 0 (no -0).

Precision.  The scale and the quotient decide integer codes, so the oracle
takes them in IEEE float32, the precision the GPU kernel computes in (numpy's
float32 division is correctly rounded); the rounding of the float32 quotient
to the code grid is then exact (formats.rne / rint in float64 on a float32
value).  Inputs are fp16 / bf16 values, hence exact in float32.
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_encode, e2m1_value, e4m3_encode, e4m3_value, e8m0_value, int8_value, ulp

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
    v = (x32 / s[:, None]).astype(np.float32)             # float32 quotient, correctly rounded
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
    element (plus 2^-22 relative for the float32 quotient)."""
    s = np.asarray(scales, dtype=np.float64)[:, None]
    v = np.abs(np.asarray(x, dtype=np.float64)) / s
    half = 0.5 * ulp(np.minimum(v, Q_FP8), "e4m3") if out == "fp8" else np.full_like(v, 0.5)
    return (half + 2.0 ** -22 * v) * s


# ----------------------------------------------------------------------------
# MXFP4 activations (for W4A4: MXFP4 weights x MXFP4 activations)
# ----------------------------------------------------------------------------
#
# Source: the OCP Microscaling (MX) v1.0 specification, section on converting
# a vector of scalars to an MX block: the shared exponent of a block of 32 is
# floor(log2(max |v|)) minus the element format's largest exponent (2 for
# E2M1, whose largest value is 6 = 1.5 * 2^2), stored as the E8M0 code
# X + 127; each element is v / 2^X rounded to E2M1 (ties to even), saturated
# to +-6.  The pages list MXFP4 among the weight formats (cocoloop.cn, format
# section) and W4A4 is the survey's next row; the rule for activations is the
# specification's.  Readings: an all-zero block takes X = 0 (code 127) with
# zero elements; X is clamped to [-127, 127]; a value that rounds to zero
# gives code 0.  Division by 2^X is exact, so no float32 decision is involved.

E2M1_EMAX = 2


def mx_quantize_rows(x, block: int = 32):
    """MXFP4 quantisation of the rows of x (float array [m, k], k % 32 == 0).

    Returns (codes uint8 [m, k] holding 0..15, e8m0 uint8 [m, k/32])."""
    x = np.asarray(x, dtype=np.float64)
    m, k = x.shape
    if k % block:
        raise ValueError("k must be a multiple of the block size")
    xb = x.reshape(m, k // block, block)
    amax = np.max(np.abs(xb), axis=2)
    safe = np.where(amax > 0, amax, 1.0)
    _, E = np.frexp(safe)                          # amax = f * 2^E, f in [0.5, 1): floor(log2) = E - 1
    X = np.where(amax > 0, (E - 1) - E2M1_EMAX, 0)
    X = np.clip(X, -127, 127).astype(np.int64)
    v = xb / np.ldexp(1.0, X)[:, :, None]          # exact: a power-of-two scaling
    codes = e2m1_encode(np.clip(v, -6.0, 6.0)).reshape(m, k)
    return codes, (X + 127).astype(np.uint8)


def mx_values(codes, e8m0, block: int = 32) -> np.ndarray:
    """e2m1(code) * 2^(X - 127) in float64 ([m, k] codes, [m, k/32] scales)."""
    c = np.asarray(codes)
    val = e2m1_value(c)
    sc = e8m0_value(np.asarray(e8m0))
    return val * np.repeat(sc, block, axis=1)
