"""Seeded synthetic inputs for the quantized GEMM workloads.

This module only draws random numbers and stores them in the canonical input
formats (packed codes, fp16/bf16/fp8 tensors).  It holds none of the GEMM's
arithmetic and is the one piece shared by the CPU oracle (``oracle``) and the
GPU library's tests and benchmark.

Recipe (every tensor drawn from ``numpy.random.default_rng`` seeded by a
SeedSequence of the workload key, in this fixed order: A, codes, scales,
zeros | E8M0, router logits):

* A: standard normal, rounded to fp16 / bf16 (round-to-nearest-even).  For the
  8-bit activation paths A is drawn the same way in fp32 and quantised per
  token: s = max|a| / 448 (fp8 e4m3) or max|a| / 127 (int8), codes =
  RNE(clamp(a / s)).  Codes and scales are then the inputs.
* Weight codes: uint4 uniform over [0, 15], packed 8 per int32 along K, code
  k = 8j + i in bits [4i, 4i+4) of word j.
* Group scales (group 128 along K): uniform in [0.005, 0.02], rounded to the
  scale dtype.  Zero points: fixed 8, or uint4 uniform in [6, 9].
* MXFP4: E2M1 codes uniform over all 16 codes; E8M0 block scales (one per 32
  along K) with exponents uniform over the integers -8..-4 (codes 119..123).
* MoE: router logits standard normal [T, E]; routing = top-k of the softmax
  (float64), weights not renormalised; expert weights drawn expert by expert
  so host memory stays bounded.
"""
from __future__ import annotations

import numpy as np
import torch

GROUP = 128
MX_BLOCK = 32


def rng_for(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def pack_u4(q: np.ndarray) -> np.ndarray:
    """uint8 codes [..., K] (values 0..15) -> int32 words [..., K/8]."""
    q = np.asarray(q, dtype=np.uint32)
    if q.shape[-1] % 8:
        raise ValueError("K must be a multiple of 8")
    q = q.reshape(q.shape[:-1] + (q.shape[-1] // 8, 8))
    w = np.zeros(q.shape[:-1], dtype=np.uint32)
    for i in range(8):
        w |= q[..., i] << np.uint32(4 * i)
    return w.view(np.int32)


def _to_dtype(x64: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float64 draw -> fp32 (RNE) -> target dtype (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(dtype)


def quant_per_token(a32: torch.Tensor, kind: str):
    """Per-token absmax quantisation of an fp32 [M, K] tensor (input prep)."""
    amax = a32.abs().amax(dim=1)
    if kind == "fp8":
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        codes = (a32 / s[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        return codes.view(torch.uint8), s.float()
    if kind == "int8":
        s = torch.where(amax > 0, amax / 127.0, torch.ones_like(amax))
        codes = torch.round(a32 / s[:, None]).clamp(-127, 127).to(torch.int8)
        return codes, s.float()
    raise ValueError(kind)


def _dtype(name: str) -> torch.dtype:
    return {"f16": torch.float16, "bf16": torch.bfloat16}[name]


def dense_w4a16(M: int, N: int, K: int, act: str = "f16", zp: str = "fixed", key=(0,)):
    """Dense W4A16 inputs.  zp: 'fixed' (zero 8) or 'u4' (per group, [6, 9])."""
    rng = rng_for(*key, M, N, K)
    dt = _dtype(act)
    a = _to_dtype(rng.standard_normal((M, K)), dt)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    scales = _to_dtype(rng.uniform(0.005, 0.02, size=(N, K // GROUP)), dt)
    zeros = None
    if zp == "u4":
        zeros = rng.integers(6, 10, size=(N, K // GROUP), dtype=np.uint8)
    return {"a": a, "codes": pack_u4(q), "scales": scales, "zeros": zeros, "act": act}


def dense_w8a16(M: int, N: int, K: int, act: str = "bf16", key=(7,)):
    """Dense W8A16 inputs: INT8 codes uniform over 0..255 (uint8 [N, K]), zero 128."""
    rng = rng_for(*key, M, N, K)
    dt = _dtype(act)
    a = _to_dtype(rng.standard_normal((M, K)), dt)
    q = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    scales = _to_dtype(rng.uniform(0.0005, 0.002, size=(N, K // GROUP)), dt)
    return {"a": a, "codes": q, "scales": scales}


def dense_w2a16(M: int, N: int, K: int, act: str = "bf16", key=(8,)):
    """Dense W2A16 inputs: uniformly random int32 words [N, K/16] (every 2-bit
    code uniform over 0..3), zero 2."""
    rng = rng_for(*key, M, N, K)
    dt = _dtype(act)
    a = _to_dtype(rng.standard_normal((M, K)), dt)
    words = rng.integers(0, 1 << 32, size=(N, K // 16), dtype=np.uint64).astype(np.uint32).view(np.int32)
    scales = _to_dtype(rng.uniform(0.01, 0.04, size=(N, K // GROUP)), dt)
    return {"a": a, "codes": words, "scales": scales}


def dense_w3a16(M: int, N: int, K: int, act: str = "bf16", key=(9,)):
    """Dense W3A16 inputs: uniformly random int32 words [N, 3K/32] (every 3-bit
    code of the bit stream uniform over 0..7), zero 4."""
    rng = rng_for(*key, M, N, K)
    dt = _dtype(act)
    a = _to_dtype(rng.standard_normal((M, K)), dt)
    words = rng.integers(0, 1 << 32, size=(N, K // 32 * 3), dtype=np.uint64).astype(np.uint32).view(np.int32)
    scales = _to_dtype(rng.uniform(0.005, 0.02, size=(N, K // GROUP)), dt)
    return {"a": a, "codes": words, "scales": scales}


def w4a16_mxint4(M: int, N: int, K: int, act: str = "bf16", key=(10,)):
    """W4A16-MXINT4 inputs: 16-bit A, MXINT4 codes uniform over 0..15 (packed as
    INT4), E8M0 block scales 2^-6..2^-2."""
    rng = rng_for(*key, M, N, K)
    a = _to_dtype(rng.standard_normal((M, K)), _dtype(act))
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    e8 = (127 + rng.integers(-6, -1, size=(N, K // MX_BLOCK))).astype(np.uint8)
    return {"a": a, "codes": pack_u4(q), "e8m0": e8}


def w4a16_nvfp4(M: int, N: int, K: int, act: str = "bf16", key=(11,)):
    """W4A16-NVFP4 inputs: 16-bit A, E2M1 codes uniform over 0..15, positive E4M3
    block scales with exponents 2^-4..2^0 and any mantissa, tensor scale 0.75."""
    rng = rng_for(*key, M, N, K)
    a = _to_dtype(rng.standard_normal((M, K)), _dtype(act))
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    e4 = ((rng.integers(3, 8, size=(N, K // 16)) << 3) | rng.integers(0, 8, size=(N, K // 16))).astype(np.uint8)
    return {"a": a, "codes": pack_u4(q), "e4m3": e4, "tscale": np.array([0.75], np.float32)}


def w4a8_mxfp4(M: int, N: int, K: int, key=(3,)):
    """W4A8-MXFP4 inputs: fp8 e4m3 per-token A, E2M1 codes, E8M0 block scales."""
    rng = rng_for(*key, M, N, K)
    a32 = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    a_codes, a_scale = quant_per_token(a32, "fp8")
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    e8 = (127 + rng.integers(-8, -3, size=(N, K // MX_BLOCK))).astype(np.uint8)
    return {"a_codes": a_codes, "a_scale": a_scale, "codes": pack_u4(q), "e8m0": e8}


def w4a4_mxfp4(M: int, N: int, K: int, key=(6,)):
    """W4A4-MXFP4 inputs: E2M1 activation codes (packed like the weights) with
    E8M0 block scales 2^-2..2^1, E2M1 weight codes with E8M0 scales 2^-8..2^-4."""
    rng = rng_for(*key, M, N, K)
    qa = rng.integers(0, 16, size=(M, K), dtype=np.uint8)
    ea = (127 + rng.integers(-2, 2, size=(M, K // MX_BLOCK))).astype(np.uint8)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    e8 = (127 + rng.integers(-8, -3, size=(N, K // MX_BLOCK))).astype(np.uint8)
    return {"a_codes": pack_u4(qa), "a_e8m0": ea, "codes": pack_u4(q), "e8m0": e8}


def w4a8_int(M: int, N: int, K: int, key=(4,)):
    """W4A8-INT inputs: int8 per-token A, symmetric INT4 codes, fp16 scales."""
    rng = rng_for(*key, M, N, K)
    a32 = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    a_codes, a_scale = quant_per_token(a32, "int8")
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    scales = _to_dtype(rng.uniform(0.005, 0.02, size=(N, K // GROUP)), torch.float16)
    return {"a_codes": a_codes, "a_scale": a_scale, "codes": pack_u4(q), "scales": scales}


def route(logits: np.ndarray, topk: int):
    """softmax (float64) + top-k, ties broken by the lower expert index."""
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.lexsort((np.broadcast_to(np.arange(p.shape[1]), p.shape), -p), axis=1)
    ids = order[:, :topk]
    w = np.take_along_axis(p, ids, axis=1)
    if topk < p.shape[1]:
        nxt = np.take_along_axis(p, order[:, topk : topk + 1], axis=1)
        if np.any(nxt[:, 0] == w[:, -1]):
            raise ValueError("tie at the top-k boundary")
    return ids.astype(np.int32), w.astype(np.float32)


def moe_routing(T: int, E: int = 256, topk: int = 8, key=(5,)):
    rng = rng_for(*key, T, E, topk, 1)
    logits = rng.standard_normal((T, E))
    ids, w = route(logits, topk)
    return {"topk_ids": ids, "topk_w": w}


def moe_activations(T: int, H: int = 7168, act: str = "bf16", key=(5,)):
    rng = rng_for(*key, T, H, 2)
    x = rng.standard_normal((T, H))
    if act in ("bf16", "f16"):
        return {"x": _to_dtype(x, torch.bfloat16 if act == "bf16" else torch.float16)}
    codes, s = quant_per_token(torch.from_numpy(x.astype(np.float32)), "fp8")
    return {"x_codes": codes, "x_scale": s}


def moe_weights(E: int = 256, H: int = 7168, I: int = 256, key=(5,), experts=None, zp: str = "fixed"):
    """Expert weights, drawn expert by expert.  W1 [E, 2I, H/8], W2 [E, H, I/8].

    ``experts`` restricts the draw to a subset (others left zero) while keeping
    every drawn expert identical to a full draw: each expert has its own seed.
    zp "u4" adds per-group uint4 zero points z1 [E, 2I, H/128], z2 [E, H, I/128]
    (uniform 6..9, drawn after the codes and scales from a seed of their own).
    """
    w1 = np.zeros((E, 2 * I, H // 8), dtype=np.int32)
    s1 = torch.zeros((E, 2 * I, H // GROUP), dtype=torch.float16)
    w2 = np.zeros((E, H, I // 8), dtype=np.int32)
    s2 = torch.zeros((E, H, I // GROUP), dtype=torch.float16)
    for e in range(E) if experts is None else sorted(set(int(x) for x in experts)):
        rng = rng_for(*key, E, H, I, 3, e)
        w1[e] = pack_u4(rng.integers(0, 16, size=(2 * I, H), dtype=np.uint8))
        s1[e] = _to_dtype(rng.uniform(0.005, 0.02, size=(2 * I, H // GROUP)), torch.float16)
        w2[e] = pack_u4(rng.integers(0, 16, size=(H, I), dtype=np.uint8))
        s2[e] = _to_dtype(rng.uniform(0.005, 0.02, size=(H, I // GROUP)), torch.float16)
    out = {"w1": w1, "s1": s1, "w2": w2, "s2": s2}
    if zp == "u4":
        z1 = np.zeros((E, 2 * I, H // GROUP), dtype=np.uint8)
        z2 = np.zeros((E, H, I // GROUP), dtype=np.uint8)
        for e in range(E) if experts is None else sorted(set(int(x) for x in experts)):
            rng = rng_for(*key, E, H, I, 4, e)
            z1[e] = rng.integers(6, 10, size=(2 * I, H // GROUP), dtype=np.uint8)
            z2[e] = rng.integers(6, 10, size=(H, I // GROUP), dtype=np.uint8)
        out.update(z1=z1, z2=z2)
    return out
