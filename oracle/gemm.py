"""Dense quantized-GEMM oracles (test infrastructure only).

Each oracle is the definition written out: unpack the codes one nibble at a
time, dequantise each weight exactly in float64, and form C = A . W_deq^T with
a float64 matrix product.  No blocking, fusion or reordering beyond that.

Sources.  Humming: open-source kernel library for quantized inference
(news.ditty.ir), summary: weights, scales and zero points are described as
separate parameters of one unified format, and the library covers WnA16 and
W4A8 (including W4A8-MXFP4, where FP8 activations meet MXFP4 weights).
cocoloop.cn (vi/fr), format section: MXFP4 is a supported weight format.
The arithmetic of each format comes from its specification (formats.py).

Readings where the pages are silent:

* Dequantisation is w = (q - z) * s with the integer zero point subtracted
  before scaling; group g covers k in [G*g, G*g + G) for every row n.
* Scales and zero points are row-major [N, K/G], n-major like the codes.
* A symmetric INT4 weight (fixed zero 8) stands for q - 8 in [-8, 7].
* INT8 weights (WnA16 with n = 8; the pages list INT1..INT8 widths): one
  unsigned byte per weight with a fixed zero point (128 for the symmetric
  case), w = (q - z) * s with group-128 scales as for INT4.
* INT2 weights (n = 2): 16 codes per int32 along K, code k = 16j + i in bits
  [2i, 2i+2) of word j, a fixed zero point 0..3 (2 for the symmetric case),
  w = (q - z) * s with group-128 scales.
* INT3 weights (n = 3; GPTQ INT3 is the named case): the dense 3-bit packing
  along K, 32 codes per 3 int32 words, code k in bits [3k, 3k+3) of the row's
  little-endian bit stream (so codes 10 and 21 of every 32 straddle two
  words), a fixed zero point 0..7 (4 for the symmetric case),
  w = (q - z) * s with group-128 scales.
* MXINT4 weights (the pages list MXINT4 among the formats): 4-bit
  two's-complement elements with an implicit 2^-2 (formats.mxint4_value),
  one E8M0 scale 2^(X-127) per 32 k as for MXFP4; with fp16/bf16
  activations C = A . W^T, W exact in float64.
* NVFP4 weights (the pages list NVFP4 among the formats): E2M1 elements,
  one FP8 E4M3 scale per 16 k and one float32 scale per tensor (NVIDIA's
  published definition of the format); w = e2m1(q) * e4m3(s_b) * s_t, exact
  in float64; with fp16/bf16 activations C = A . W^T.
* W4A8-INT: the int32 accumulator of one group is
  P[m,n,g] = sum_{k in g} a_q[m,k] * (q[n,k] - 8), and
  C = s_a[m] * sum_g s[n,g] * P[m,n,g].
* W4A8-MXFP4: C = s_a[m] * sum_k e4m3(a_q[m,k]) * e2m1(q[n,k]) * 2^(E[n,k/32]-127).
  The inner sum is a sum of multiples of 2^-18 below 2^21 in magnitude at
  these sizes, so it is exact in float64 in any order.
* Tolerance per output: tau = 1e-2 * (sum_k |a*w|) / K * sqrt(K), plus half
  an output ulp (the rounding of the result to fp16/bf16 that every
  implementation, this oracle included, must incur).
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_value, e4m3_value, e8m0_value, int8_value, mxint4_value, rne, ulp, unpack_u4


def dequant_int4(codes, scales, zeros, group: int = 128) -> np.ndarray:
    """Exact float64 weights w[n,k] = (q[n,k] - z[n,k//G]) * s[n,k//G].

    codes  int32 [N, K/8] (canonical packing)
    scales float array-like [N, K/G] (the fp16/bf16 values, widened exactly)
    zeros  None -> 8 (symmetric), an int -> that fixed zero, or an integer
           array [N, K/G] of per-group zero points.
    """
    q = unpack_u4(codes).astype(np.int64)
    N, K = q.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    s = np.asarray(scales, dtype=np.float64)
    if zeros is None:
        z = np.full(s.shape, 8, dtype=np.int64)
    elif np.isscalar(zeros):
        z = np.full(s.shape, int(zeros), dtype=np.int64)
    else:
        z = np.asarray(zeros).astype(np.int64)
    w = np.empty((N, K), dtype=np.float64)
    for g in range(K // group):
        ks = slice(g * group, (g + 1) * group)
        w[:, ks] = (q[:, ks] - z[:, g : g + 1]) * s[:, g : g + 1]
    return w


def tolerance(a, w) -> np.ndarray:
    """tau[m,n] = 1e-2 * (sum_k |a[m,k] w[n,k]|) / K * sqrt(K), in float64."""
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    K = a.shape[1]
    return 1e-2 * (np.abs(a) @ np.abs(w).T) / K * np.sqrt(K)


def check(c_gpu, c64, tau, out_fmt: str):
    """Per-output pass mask: |c_gpu - c64| <= tau + ulp_out(max(|c_gpu|,|c64|))/2.

    Returns (ok, literal_ok, err_over_tau).  ``literal_ok`` is the bare
    |err| <= tau check, reported alongside.
    """
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    err = np.abs(c_gpu - c64)
    half = 0.5 * ulp(np.maximum(np.abs(c_gpu), np.abs(c64)), out_fmt)
    ok = err <= tau + half
    ok &= np.isfinite(c_gpu)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tau > 0, err / tau, np.where(err == 0, 0.0, np.inf))
    return ok, err <= tau, ratio


def gemm_w4a16(a, codes, scales, zeros=None, group: int = 128, out_fmt: str = "f16"):
    """Dense W4A16: C = A . ((q - z) * s)^T, float64 accumulate.

    a  float array [M, K] holding the fp16/bf16 activation values exactly.
    Returns dict(c64, c_out (rounded to out_fmt), tau).
    """
    a = np.asarray(a, dtype=np.float64)
    w = dequant_int4(codes, scales, zeros, group)
    c64 = a @ w.T
    return {"c64": c64, "c_out": rne(c64, out_fmt), "tau": tolerance(a, w), "w": w}


def dequant_int8(codes, scales, zero: int = 128, group: int = 128) -> np.ndarray:
    """Exact float64 weights w[n,k] = (q[n,k] - z) * s[n,k//G] for 8-bit codes.

    codes  uint8 [N, K] (canonical: one byte per weight, row-major; an int32
           [N, K/4] array of the same bytes, low byte first, is accepted)
    scales float array-like [N, K/G]; zero the fixed zero point 0..255.
    """
    c = np.ascontiguousarray(codes)
    q = (c.view(np.uint8) if c.dtype != np.uint8 else c).astype(np.int64)
    N, K = q.shape[0], q.size // q.shape[0]
    q = q.reshape(N, K)
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    s = np.asarray(scales, dtype=np.float64)
    w = np.empty((N, K), dtype=np.float64)
    for g in range(K // group):
        ks = slice(g * group, (g + 1) * group)
        w[:, ks] = (q[:, ks] - int(zero)) * s[:, g : g + 1]
    return w


def unpack_u2(words) -> np.ndarray:
    """Unpack int32 words [..., K/16] into 2-bit codes [..., K]: code k = 16j + i
    sits in bits [2i, 2i+2) of word j (low bits first)."""
    w = np.ascontiguousarray(words).view(np.uint32)
    out = np.empty(w.shape[:-1] + (w.shape[-1] * 16,), dtype=np.uint8)
    for i in range(16):
        out[..., i::16] = (w >> np.uint32(2 * i)) & np.uint32(0x3)
    return out


def dequant_int2(codes, scales, zero: int = 2, group: int = 128) -> np.ndarray:
    """Exact float64 weights w[n,k] = (q[n,k] - z) * s[n,k//G] for 2-bit codes
    (int32 [N, K/16] canonical packing), fixed zero point z in 0..3."""
    q = unpack_u2(codes).astype(np.int64)
    N, K = q.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    s = np.asarray(scales, dtype=np.float64)
    w = np.empty((N, K), dtype=np.float64)
    for g in range(K // group):
        ks = slice(g * group, (g + 1) * group)
        w[:, ks] = (q[:, ks] - int(zero)) * s[:, g : g + 1]
    return w


def unpack_u3(words) -> np.ndarray:
    """Unpack int32 words [..., 3K/32] into 3-bit codes [..., K].  The words of a
    row form one little-endian bit stream (word j holds stream bits [32j, 32j+32),
    lowest first) and code k is the 3-bit number at stream bits [3k, 3k+3), so
    32 codes fill 3 words and some codes straddle two words: the dense 3-bit
    packing along K of GPTQ INT3 checkpoints."""
    w = np.ascontiguousarray(words).view(np.uint32)
    if w.shape[-1] % 3:
        raise ValueError("INT3 rows hold a multiple of 3 words (32 codes per 3 words)")
    le = np.ascontiguousarray(w.astype("<u4")).view(np.uint8)  # bytes in stream order
    bits = np.unpackbits(le, axis=-1, bitorder="little")  # stream bit b at index b
    K = bits.shape[-1] // 3
    b = bits.reshape(w.shape[:-1] + (K, 3))
    return (b[..., 0] | (b[..., 1] << 1) | (b[..., 2] << 2)).astype(np.uint8)


def dequant_int3(codes, scales, zero: int = 4, group: int = 128) -> np.ndarray:
    """Exact float64 weights w[n,k] = (q[n,k] - z) * s[n,k//G] for 3-bit codes
    (int32 [N, 3K/32] bit-stream packing), fixed zero point z in 0..7."""
    q = unpack_u3(codes).astype(np.int64)
    N, K = q.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    s = np.asarray(scales, dtype=np.float64)
    w = np.empty((N, K), dtype=np.float64)
    for g in range(K // group):
        ks = slice(g * group, (g + 1) * group)
        w[:, ks] = (q[:, ks] - int(zero)) * s[:, g : g + 1]
    return w


def gemm_w3a16(a, codes, scales, zero: int = 4, group: int = 128, out_fmt: str = "f16"):
    """Dense W3A16 (INT3 weights, one of the WnA16 widths): C = A . ((q - z) * s)^T, float64."""
    a = np.asarray(a, dtype=np.float64)
    w = dequant_int3(codes, scales, zero, group)
    c64 = a @ w.T
    return {"c64": c64, "c_out": rne(c64, out_fmt), "tau": tolerance(a, w), "w": w}


def gemm_w2a16(a, codes, scales, zero: int = 2, group: int = 128, out_fmt: str = "f16"):
    """Dense W2A16 (INT2 weights, one of the WnA16 widths): C = A . ((q - z) * s)^T, float64."""
    a = np.asarray(a, dtype=np.float64)
    w = dequant_int2(codes, scales, zero, group)
    c64 = a @ w.T
    return {"c64": c64, "c_out": rne(c64, out_fmt), "tau": tolerance(a, w), "w": w}


def gemm_w8a16(a, codes, scales, zero: int = 128, group: int = 128, out_fmt: str = "f16"):
    """Dense W8A16 (INT8 weights, one of the WnA16 widths): C = A . ((q - z) * s)^T, float64."""
    a = np.asarray(a, dtype=np.float64)
    w = dequant_int8(codes, scales, zero, group)
    c64 = a @ w.T
    return {"c64": c64, "c_out": rne(c64, out_fmt), "tau": tolerance(a, w), "w": w}


def mxfp4_weights(codes, e8m0, block: int = 32) -> np.ndarray:
    """w[n,k] = e2m1(q[n,k]) * 2^(E[n, k//32] - 127), exact in float64."""
    q = unpack_u4(codes)
    N, K = q.shape
    scale = e8m0_value(np.asarray(e8m0))
    if scale.shape != (N, K // block):
        raise ValueError("E8M0 scales must be [N, K/32]")
    w = e2m1_value(q)
    for b in range(K // block):
        w[:, b * block : (b + 1) * block] *= scale[:, b : b + 1]
    return w


def mxint4_weights(codes, e8m0, block: int = 32) -> np.ndarray:
    """w[n,k] = mxint4(q[n,k]) * 2^(E[n, k//32] - 127), exact in float64."""
    q = unpack_u4(codes)
    N, K = q.shape
    scale = e8m0_value(np.asarray(e8m0))
    if scale.shape != (N, K // block):
        raise ValueError("E8M0 scales must be [N, K/32]")
    w = mxint4_value(q)
    for b in range(K // block):
        w[:, b * block : (b + 1) * block] *= scale[:, b : b + 1]
    return w


def gemm_mxint4_w16(a, w_codes, e8m0, out_fmt: str = "bf16"):
    """W4A16-MXINT4: C = A . W^T with fp16/bf16 activation values A and the
    MXINT4 weights (mxint4_weights), float64."""
    a = np.asarray(a, dtype=np.float64)
    w = mxint4_weights(w_codes, e8m0)
    c64 = a @ w.T
    return {"c64": c64, "c_out": rne(c64, out_fmt), "tau": tolerance(a, w), "w": w}


def nvfp4_weights(codes, e4m3_scales, tensor_scale, block: int = 16) -> np.ndarray:
    """w[n,k] = e2m1(q[n,k]) * e4m3(S[n, k//16]) * s_t, exact in float64."""
    q = unpack_u4(codes)
    N, K = q.shape
    sb = e4m3_value(np.asarray(e4m3_scales))
    if sb.shape != (N, K // block):
        raise ValueError("E4M3 block scales must be [N, K/16]")
    w = e2m1_value(q)
    for b in range(K // block):
        w[:, b * block : (b + 1) * block] *= sb[:, b : b + 1]
    return w * float(tensor_scale)


def gemm_nvfp4_w16(a, w_codes, e4m3_scales, tensor_scale, out_fmt: str = "bf16"):
    """W4A16-NVFP4: C = A . W^T with fp16/bf16 activation values A and the
    NVFP4 weights (nvfp4_weights), float64."""
    a = np.asarray(a, dtype=np.float64)
    w = nvfp4_weights(w_codes, e4m3_scales, tensor_scale)
    c64 = a @ w.T
    return {"c64": c64, "c_out": rne(c64, out_fmt), "tau": tolerance(a, w), "w": w}


def gemm_mxfp4_fp8(a_codes, a_scale, w_codes, e8m0, out_fmt: str = "bf16"):
    """W4A8-MXFP4: C[m,n] = s_a[m] * sum_k e4m3(a_q[m,k]) * w[n,k]."""
    a = e4m3_value(np.asarray(a_codes))
    sa = np.asarray(a_scale, dtype=np.float64)
    w = mxfp4_weights(w_codes, e8m0)
    inner = a @ w.T  # exact: see module docstring
    c64 = sa[:, None] * inner
    a_val = a * sa[:, None]
    return {"c64": c64, "c_out": rne(c64, out_fmt), "tau": tolerance(a_val, w), "w": w}


def gemm_mxfp4_mxfp4(a_codes, a_e8m0, w_codes, w_e8m0, out_fmt: str = "bf16"):
    """W4A4-MXFP4: C[m,n] = sum_k e2m1(qa[m,k]) 2^(Xa[m,k/32]-127) * e2m1(qw[n,k]) 2^(Xw[n,k/32]-127).

    a_codes int32 [M, K/8] (canonical packing, like the weights), a_e8m0
    uint8 [M, K/32].  Every product is a multiple of 2^(Xa+Xw-256) below
    2^(Xa+Xw-248) in magnitude; with the scale ranges of these workloads the
    float64 sum is exact in any order."""
    a = mxfp4_weights(a_codes, a_e8m0)  # the activation block format is the weights' one
    w = mxfp4_weights(w_codes, w_e8m0)
    c64 = a @ w.T
    return {"c64": c64, "c_out": rne(c64, out_fmt), "tau": tolerance(a, w), "w": w}


def int_accumulators(a_codes, w_codes, group: int = 128) -> np.ndarray:
    """P[m,n,g] = sum_{k in g} a_q[m,k] * (q[n,k] - 8), exact int64."""
    a = int8_value(np.asarray(a_codes)).astype(np.int64)
    wq = unpack_u4(w_codes).astype(np.int64) - 8
    M, K = a.shape
    N = wq.shape[0]
    G = K // group
    P = np.zeros((M, N, G), dtype=np.int64)
    for g in range(G):
        ks = slice(g * group, (g + 1) * group)
        P[:, :, g] = a[:, ks] @ wq[:, ks].T
    return P


def gemm_int4_int8(a_codes, a_scale, w_codes, scales, group: int = 128, out_fmt: str = "bf16"):
    """W4A8-INT: exact per-group int accumulators, then the float epilogue."""
    P = int_accumulators(a_codes, w_codes, group)
    s = np.asarray(scales, dtype=np.float64)  # [N, G]
    sa = np.asarray(a_scale, dtype=np.float64)
    c64 = sa[:, None] * np.einsum("mng,ng->mn", P.astype(np.float64), s)
    a_val = int8_value(np.asarray(a_codes)) * sa[:, None]
    w = dequant_int4(w_codes, scales, 8, group)
    return {"P": P, "c64": c64, "c_out": rne(c64, out_fmt), "tau": tolerance(a_val, w), "w": w}
