"""Grouped (mixture-of-experts) quantized GEMM oracle (test infrastructure only).

Sources.  Humming: open-source kernel library for quantized inference
(news.ditty.ir), summary and key points: besides the dense GEMM the library
has an MoE "Grouped" path, selected with its own backend switch, run with
W4A16 or W4A8 weights; mixture-of-experts models keep every expert's weights
in memory while each token activates only a few of them.  The pages give no
routing, layout or formula; the layer below is the plainest reading of a
DeepSeek-style expert layer (256 experts, top-8, SiLU-gated MLP) restricted to
one GPU's tensor-parallel share.

Readings (listed with the rest in the design notes):

* Routing ids [T, topk] and weights [T, topk] are inputs (softmax of router
  logits, top-k, not renormalised -- made by the input generator).
* Expert e's first GEMM W1_e has 2*I rows: rows [0, I) are the gate, rows
  [I, 2I) the up projection; act = SiLU(gate) * up, SiLU(x) = x / (1 + e^-x).
* W4A16: act is rounded to bf16.  W4A8: act is requantised per (token, slot)
  row to fp8 e4m3 with s = max|act| / 448, codes = RNE_e4m3(act / s).
* The top-k weight multiplies each down-projection row in float before the
  sum over slots: y_t = sum_j w[t,j] * (act_{t,j} . W2_{e_j}^T), rounded to bf16.
* Each stage is checked on the GPU's own input to that stage, so that a one-ulp
  flip in a requantised code does not cascade into the next stage.
* Where the weighted slot rows are stored in bf16 before the sum over a
  token's slots, each is a GEMM output with its own output rounding, and the
  bound on y grows by that rounding (``rows_rounding_bound``).

Align ("moe_align") has many correct results (any order inside an expert's
segment); ``check_align`` verifies the invariants rather than an array.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_value, rne, ulp
from .gemm import dequant_int4, tolerance


def check_align(topk_ids, num_experts: int, block_m: int, sorted_ids, block_expert, num_padded):
    """Raise AssertionError unless (sorted_ids, block_expert, num_padded) is a
    valid expert alignment of ``topk_ids`` with blocks of ``block_m`` rows.

    Valid means: the non-sentinel entries of sorted_ids[:num_padded] are a
    permutation of the flat slots 0..T*topk-1; every block holds slots of one
    segment only; the segments are the experts 0..E-1 in increasing order and
    then one segment for ids outside [0, E) (block_expert -1); a segment with
    c slots occupies exactly ceil(c / block_m) consecutive blocks; every other
    entry in [0, num_padded) is the sentinel T*topk.  (The pages do not
    describe the routing data structures; this is the layout the grouped GEMM
    needs: each expert's slots contiguous and padded to whole row blocks.)
    """
    ids = np.asarray(topk_ids).astype(np.int64)
    T, topk = ids.shape
    flat = ids.reshape(-1)
    seg = np.where((flat >= 0) & (flat < num_experts), flat, num_experts)  # segment of each slot
    sentinel = T * topk
    npad = int(np.asarray(num_padded).reshape(-1)[0])
    sid = np.asarray(sorted_ids).astype(np.int64)[:npad]
    bexp = np.asarray(block_expert).astype(np.int64)
    assert npad % block_m == 0, "num_padded is not a multiple of block_m"
    counts = np.bincount(seg, minlength=num_experts + 1)
    expect_blocks = -(-counts // block_m)
    assert npad == int(expect_blocks.sum()) * block_m, "num_padded is not the minimum padded length"
    valid = sid[sid != sentinel]
    assert np.all((sid >= 0) & (sid <= sentinel)), "sorted id out of range"
    assert valid.size == flat.size and np.array_equal(np.sort(valid), np.arange(flat.size)), \
        "sorted ids are not a permutation of the slots"
    nb = npad // block_m
    b = 0
    for e in range(num_experts + 1):
        for _ in range(int(expect_blocks[e])):
            want = e if e < num_experts else -1
            assert bexp[b] == want, f"block {b} should belong to segment {want}"
            rows = sid[b * block_m : (b + 1) * block_m]
            rows = rows[rows != sentinel]
            assert np.all(seg[rows] == e), f"block {b} holds slots of another segment"
            b += 1
    assert b == nb
    return True


def silu(x):
    """SiLU(x) = x * sigmoid(x) = x / (1 + e^-x), float64."""
    return x / (1.0 + np.exp(-x))


def silu_grad(x):
    """d/dx SiLU(x) = sigmoid(x) (1 + x (1 - sigmoid(x))), float64."""
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def grouped_gemm(rows_a, row_expert, codes, scales, zeros=8, group: int = 128):
    """out[r] = rows_a[r] . W_{e(r)}^T for each row, float64; also its tau.

    rows_a     float64 [R, K]   activation values of each (token, slot) row
    row_expert int [R]          expert of each row
    codes      int32 [E, N, K/8], scales [E, N, K/G]
    zeros      a fixed zero point, or per-group zero points [E, N, K/G]
    """
    rows_a = np.asarray(rows_a, dtype=np.float64)
    R, K = rows_a.shape
    N = codes.shape[1]
    out = np.zeros((R, N))
    tau = np.zeros((R, N))
    for e in np.unique(row_expert):
        sel = np.nonzero(row_expert == e)[0]
        w = dequant_int4(codes[e], scales[e], zeros if np.isscalar(zeros) else np.asarray(zeros)[e], group)
        out[sel] = rows_a[sel] @ w.T
        tau[sel] = tolerance(rows_a[sel], w)
    return out, tau


def gate_up(rows_a, row_expert, w1_codes, w1_scales, inter: int, w1_zeros=8):
    """First expert GEMM + SiLU*mul, float64, with first-order bounds.

    Returns dict(g, u, act, tau_g, tau_u, tau_act) where tau_act bounds
    |act(g + dg, u + du) - act(g, u)| for |dg| <= tau_g, |du| <= tau_u
    (first-order terms plus the Taylor remainder, SiLU'' being <= 1/2).
    """
    h, tau_h = grouped_gemm(rows_a, row_expert, w1_codes, w1_scales, w1_zeros)
    g, u = h[:, :inter], h[:, inter:]
    tg, tu = tau_h[:, :inter], tau_h[:, inter:]
    act = silu(g) * u
    return {"g": g, "u": u, "act": act, "tau_g": tg, "tau_u": tu, "tau_act": act_bound(g, u, tg, tu)}


def act_bound(g, u, tg, tu):
    """Bound on |SiLU(g + dg)(u + du) - SiLU(g) u| over |dg| <= tg, |du| <= tu.

    Writing the difference as [SiLU(g + dg) - SiLU(g)](u + du) + SiLU(g) du
    and expanding SiLU to second order with |SiLU''| <= 1/2 and |SiLU'| <= 1.1:
    |SiLU'(g) u| tg + |SiLU(g)| tu + 1.1 tg tu + (1/4) tg^2 (|u| + tu).
    """
    return (np.abs(silu_grad(g) * u) * tg + np.abs(silu(g)) * tu
            + 1.1 * tg * tu + 0.25 * tg * tg * (np.abs(u) + tu))


def requant_fp8_rows(act):
    """Per-row fp8 e4m3 requantisation (float64 statement of the reading).

    s = max|act| / 448 (s = 1 for an all-zero row); codes = RNE_e4m3(act / s)
    clamped to [-448, 448].  Returns (dequantised values, s).
    """
    act = np.asarray(act, dtype=np.float64)
    amax = np.max(np.abs(act), axis=1)
    s = np.where(amax > 0, amax / 448.0, 1.0)
    v = np.clip(act / s[:, None], -448.0, 448.0)
    return rne(v, "e4m3") * s[:, None], s


def fp8_rows_bound(dq_gpu, scale_gpu, act64, tau_act):
    """Bound for a GPU-requantised row: |codes*s - act64| <= tau_act + s*ulp_e4m3/2.

    The GPU value h = act64 + d with |d| <= tau_act is rounded on the e4m3 grid
    of h/s; the half-step is taken at the larger of the two magnitudes.  A
    relative 2^-20 allowance covers the fp32 division h/s.
    """
    s = np.asarray(scale_gpu, dtype=np.float64)[:, None]
    mag = np.maximum(np.abs(dq_gpu), np.abs(act64)) / s
    return tau_act + 0.5 * ulp(mag, "e4m3") * s + 2.0 ** -20 * np.abs(act64)


def rows_rounding_bound(o, tau_o, weight, topk: int, fmt: str = "bf16"):
    """Bound on what rounding each weighted slot row to ``fmt`` adds to y.

    Reading: where the down GEMM stores its per-slot rows in a 16-bit format
    before the sum over the token's slots, those rows are GEMM outputs like
    any other and carry their own output rounding (the tolerance rule is per
    output of a GEMM with fp16/bf16 outputs).  The GPU's weighted row is
    x = fl32(w * o_gpu) with |o_gpu - o| <= tau_o, so |x| <= B = |w| (|o| +
    tau_o) (1 + 2^-23); rounding x to ``fmt`` moves it by at most half the
    format's spacing at B, and the fp32 sum of topk such rows in slot order
    adds at most topk 2^-23 B per row.  Returns that per-row bound, [R, N].
    """
    o = np.asarray(o, dtype=np.float64)
    B = np.abs(np.asarray(weight, dtype=np.float64))[:, None] * (np.abs(o) + tau_o) * (1.0 + 2.0 ** -23)
    return 0.5 * ulp(B, fmt) + topk * 2.0 ** -23 * B


def down_combine(act_rows, row_token, row_weight, row_expert, w2_codes, w2_scales, T: int, rows_fmt=None,
                 topk: int = 8, w2_zeros=8):
    """Second expert GEMM, top-k weighting and combine, float64.

    act_rows float64 [R, I] (the GPU's own act values), row_token / row_weight
    / row_expert [R].  Returns dict(y64, tau_y) with tau_y = sum_j |w_j| tau_o
    (without the output half-ulp, which ``gemm.check`` adds), plus, when the
    weighted rows are stored in ``rows_fmt`` before the sum, the sum over the
    token's rows of ``rows_rounding_bound``.
    """
    o, tau_o = grouped_gemm(act_rows, row_expert, w2_codes, w2_scales, w2_zeros)
    H = o.shape[1]
    y = np.zeros((T, H))
    ty = np.zeros((T, H))
    wr = np.asarray(row_weight, dtype=np.float64)
    extra = rows_rounding_bound(o, tau_o, wr, topk, rows_fmt) if rows_fmt else None
    for r in range(o.shape[0]):
        t = int(row_token[r])
        y[t] += wr[r] * o[r]
        ty[t] += abs(wr[r]) * tau_o[r]
        if extra is not None:
            ty[t] += extra[r]
    return {"y64": y, "tau_y": ty, "o": o, "tau_o": tau_o}


def fp8_row_values(codes, scale):
    """Dequantised value of fp8 e4m3 row codes [R, I] with row scales [R]."""
    return e4m3_value(np.asarray(codes)) * np.asarray(scale, dtype=np.float64)[:, None]
