"""Pins of the MoE stage of the CPU oracle (oracle/moe.py) against things other
than itself (CPU only).

* SiLU at values the mathematics fixes (SiLU(0) = 0, SiLU(1) = e / (1 + e),
  SiLU(-1) = -1 / (1 + e)) and its odd-part identity SiLU(x) - SiLU(-x) = x.
* SiLU' against a central finite difference of the definition x / (1 + e^-x).
* The first-order act bound tau_act against brute-force perturbation: no
  |dg| <= tau_g, |du| <= tau_u moves SiLU(g) u by more than tau_act, and the
  bound is not loose by more than a small factor.
* The fp8 requant and its bound against a hand-worked row (e4m3 grid by hand).
* A whole two-expert layer worked by hand (tests/golden/moe_tiny.json): gate
  rows first, SiLU on the gate, top-k weights applied before the sum.
* Planted mistakes (gate and up swapped, sigmoid in place of SiLU, a sign slip
  in SiLU') each fail one of the pins.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as MO

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ SiLU ----

def _check_silu_values(silu):
    e = math.e
    assert silu(np.array([0.0]))[0] == 0.0
    assert abs(silu(np.array([1.0]))[0] - e / (1 + e)) <= 1e-15
    assert abs(silu(np.array([-1.0]))[0] + 1 / (1 + e)) <= 1e-15
    assert abs(silu(np.array([2.0]))[0] - 2 * e * e / (1 + e * e)) <= 1e-15
    x = np.random.default_rng(3).standard_normal(1000) * 6
    assert np.allclose(silu(x) - silu(-x), x, rtol=0, atol=1e-13)
    # large |x|: SiLU(x) -> x for x >> 0 and -> 0 for x << 0
    assert abs(silu(np.array([40.0]))[0] - 40.0) <= 1e-12
    assert abs(silu(np.array([-40.0]))[0]) <= 1e-15


def test_silu_fixed_values_and_odd_part():
    _check_silu_values(MO.silu)


def _check_silu_grad(silu_grad):
    # central difference of the definition x / (1 + e^-x), evaluated here in
    # exact terms of math.exp (not through the oracle's silu)
    f = lambda x: x / (1.0 + math.exp(-x))
    xs = np.concatenate([np.linspace(-8, 8, 61), [0.0, 1e-3, -1e-3]])
    h = 1e-5
    for x in xs:
        fd = (f(x + h) - f(x - h)) / (2 * h)
        g = float(silu_grad(np.array([x]))[0])
        assert abs(g - fd) <= 1e-7 * max(1.0, abs(fd)), (x, g, fd)
    # SiLU'(0) = 1/2 exactly; SiLU' lies in [-0.0999, 1.0999]
    assert silu_grad(np.array([0.0]))[0] == 0.5
    d = silu_grad(np.linspace(-20, 20, 40001))
    assert d.min() >= -0.1 and d.max() <= 1.1


def test_silu_grad_against_central_difference():
    _check_silu_grad(MO.silu_grad)


# --------------------------------------------------------------- tau_act ----

def _random_gate_up(n, seed):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(n) * 3
    u = rng.standard_normal(n) * 3
    tg = np.abs(rng.standard_normal(n)) * 0.05 + 1e-3
    tu = np.abs(rng.standard_normal(n)) * 0.05 + 1e-3
    return g, u, tg, tu


def _gate_up_bound(g, u, tg, tu):
    # oracle.moe.act_bound is the bound gate_up uses (same function)
    return MO.act_bound(g, u, tg, tu)


def test_tau_act_bounds_every_perturbation():
    n = 2000
    g, u, tg, tu = _random_gate_up(n, 5)
    tau = _gate_up_bound(g, u, tg, tu)
    act = MO.silu(g) * u
    rng = np.random.default_rng(6)
    worst = np.zeros(n)
    for _ in range(50):  # 10^5 random perturbations in the box
        dg = rng.uniform(-1, 1, n) * tg
        du = rng.uniform(-1, 1, n) * tu
        dev = np.abs(MO.silu(g + dg) * (u + du) - act)
        assert np.all(dev <= tau), "a perturbation inside the box exceeds tau_act"
        worst = np.maximum(worst, dev)
    for sg in (-1, 1):  # the box's corners
        for su in (-1, 1):
            dev = np.abs(MO.silu(g + sg * tg) * (u + su * tu) - act)
            assert np.all(dev <= tau)
            worst = np.maximum(worst, dev)
    # not loose: where the first-order terms dominate (most points) the worst
    # corner reaches nearly all of the bound, so a spurious factor of 2 fails;
    # the few points where both first-order terms vanish are bounded by the
    # worst-case second-order constants and sit lower
    r = worst / tau
    assert np.median(r) > 0.9
    assert np.quantile(r, 0.1) > 0.6


def test_tau_act_matches_gate_up_result():
    # gate_up reports the same bound for the g, u it computes
    g = _gold("moe_tiny.json")
    lay = _tiny_layer(g)
    gu = MO.gate_up(lay["rows_a"], lay["row_exp"], lay["w1"], lay["s1"], g["I"])
    assert np.allclose(gu["tau_act"], MO.act_bound(gu["g"], gu["u"], gu["tau_g"], gu["tau_u"]), rtol=0, atol=0)


# ----------------------------------------------------------- fp8 requant ----

def test_requant_fp8_rows_hand_example():
    h = _gold("moe_tiny.json")["fp8_requant"]
    act = np.array([h["act"]])
    dq, s = MO.requant_fp8_rows(act)
    assert s[0] == h["scale"]
    assert np.allclose(dq[0] / s[0], h["codes_value"], rtol=0, atol=1e-9)
    # the bound at tau_act = 0 is the half-step (times s), plus 2^-20 |act|
    b = MO.fp8_rows_bound(dq, s, act, np.zeros_like(act))
    want = np.array(h["half_step"]) * s[0] + 2.0 ** -20 * np.abs(act[0])
    assert np.allclose(b[0], want, rtol=1e-12, atol=0)
    # and every element of the hand example lies inside it
    assert np.all(np.abs(dq - act) <= b)
    # a one-step-off code (the next e4m3 value up) is outside the bound
    off = dq.copy()
    off[0, 1] = 144.0 * s[0]
    assert np.abs(off - act)[0, 1] > b[0, 1]


def test_fp8_rows_bound_covers_perturbed_requant():
    # GPU-like situation: the value requantised is act + d with |d| <= tau_act
    rng = np.random.default_rng(8)
    act = rng.standard_normal((64, 256)) * 2
    tau = np.abs(rng.standard_normal((64, 256))) * 1e-3
    h = act + rng.uniform(-1, 1, act.shape) * tau
    dq, s = MO.requant_fp8_rows(h)
    b = MO.fp8_rows_bound(dq, s, act, tau)
    assert np.all(np.abs(dq - act) <= b)


def _combine_bf16_rows(o_gpu, w, topk):
    # the aligned path's combine, simulated: x = fl32(w * o), rounded to bf16,
    # then summed in fp32 over each token's topk rows in slot order
    x = (np.float32(1) * w.astype(np.float32)[:, None] * o_gpu.astype(np.float32)).astype(np.float64)
    r = F.rne(x, "bf16").astype(np.float32)
    T = r.shape[0] // topk
    y = r[0::topk].copy()
    for j in range(1, topk):
        y = (y + r[j::topk]).astype(np.float32)
    return y.astype(np.float64).reshape(T, -1)


def test_rows_rounding_bound_covers_simulated_combine():
    rng = np.random.default_rng(10)
    topk, T, N = 8, 64, 96
    o = rng.standard_normal((T * topk, N)) * np.exp(rng.uniform(-6, 6, (T * topk, 1)))
    tau = np.abs(o) * rng.uniform(0, 1e-3, o.shape)
    w = rng.uniform(0, 1, T * topk)
    o_gpu = o + rng.uniform(-1, 1, o.shape) * tau
    y = _combine_bf16_rows(o_gpu, w, topk)
    exact = (w[:, None] * o).reshape(T, topk, N).sum(1)
    bound = (np.abs(w)[:, None] * tau + MO.rows_rounding_bound(o, tau, w, topk)).reshape(T, topk, N).sum(1)
    assert np.all(np.abs(y - exact) <= bound)


def test_rows_rounding_bound_at_midpoints_and_binade_crossings():
    # a row value exactly halfway between two bf16 values rounds by half a
    # spacing; a GPU value pushed over a power of two by its GEMM error is
    # rounded on the coarser grid above it
    topk = 1
    mid = 1.0 + 3.0 * 2.0 ** -8                            # halfway between 1 + 2^-7 and 1 + 2^-6: rounds up
    o = np.array([[1.0 + 2.0 ** -8, mid - 0.02, 3.0 * 2.0 ** -9 + 1.0]])
    tau = np.array([[0.0, 0.02, 0.0]])
    o_gpu = np.array([[1.0 + 2.0 ** -8, mid, 3.0 * 2.0 ** -9 + 1.0]])
    w = np.array([1.0])
    y = _combine_bf16_rows(o_gpu, w, topk)
    err = np.abs(y - w[:, None] * o)
    bound = np.abs(w)[:, None] * tau + MO.rows_rounding_bound(o, tau, w, topk)
    assert np.all(err <= bound)
    assert err[0, 0] == 2.0 ** -8                          # the half spacing is reached
    # planted: the spacing taken at |w o| instead of the bound on the GPU value
    planted = np.abs(w)[:, None] * tau + 0.5 * F.ulp(np.abs(w)[:, None] * np.abs(o), "bf16")
    assert not np.all(err <= planted)
    # planted: no rounding term at all
    assert not np.all(err <= np.abs(w)[:, None] * tau + topk * 2.0 ** -23 * np.abs(o))


def test_down_combine_rows_fmt_adds_the_rounding_term():
    g = _gold("moe_tiny.json")
    lay = _tiny_layer(g)
    gu = MO.gate_up(lay["rows_a"], lay["row_exp"], lay["w1"], lay["s1"], g["I"])
    plain = MO.down_combine(gu["act"], lay["row_tok"], lay["row_w"], lay["row_exp"], lay["w2"], lay["s2"], lay["T"])
    rounded = MO.down_combine(gu["act"], lay["row_tok"], lay["row_w"], lay["row_exp"], lay["w2"], lay["s2"],
                              lay["T"], rows_fmt="bf16", topk=lay["topk"])
    assert np.array_equal(plain["y64"], rounded["y64"])
    extra = MO.rows_rounding_bound(plain["o"], plain["tau_o"], lay["row_w"], lay["topk"])
    want = plain["tau_y"].copy()
    for r, t in enumerate(lay["row_tok"]):
        want[t] += extra[r]
    assert np.allclose(rounded["tau_y"], want, rtol=0, atol=0)
    assert np.all(rounded["tau_y"][np.abs(plain["y64"]) > 0] > plain["tau_y"][np.abs(plain["y64"]) > 0])


def test_fp8_scale_matches_row_maximum():
    rng = np.random.default_rng(9)
    act = rng.standard_normal((16, 256))
    act[3] = 0.0
    _, s = MO.requant_fp8_rows(act)
    want = np.abs(act).max(1) / 448.0
    want[3] = 1.0
    assert np.array_equal(s, want)


# ------------------------------------------------------ hand-worked layer ----

def _tiny_layer(g):
    H, I, E, T = g["H"], g["I"], g["E"], len(g["x"])
    w1q = np.full((E, 2 * I, H), 8, dtype=np.uint8)
    for e, r, k, c in g["w1_codes"]:
        w1q[e, r, k] = c
    w2q = np.full((E, H, I), 8, dtype=np.uint8)
    for e, r, k, c in g["w2_codes"]:
        w2q[e, r, k] = c
    pack = lambda q: _pack(q)
    x = np.zeros((T, H))
    for t, row in enumerate(g["x"]):
        for k, v in row:
            x[t, k] = v
    ids = np.array(g["topk_ids"])
    topk = ids.shape[1]
    rows_a = np.repeat(x, topk, axis=0)
    return dict(x=x, w1=pack(w1q), s1=np.ones((E, 2 * I, H // 128)), w2=pack(w2q), s2=np.ones((E, H, I // 128)),
                rows_a=rows_a, row_exp=ids.reshape(-1), row_tok=np.repeat(np.arange(T), topk),
                row_w=np.array(g["topk_w"], float).reshape(-1), T=T, topk=topk)


def _pack(q):
    # canonical packing written out here (8 codes per word, low nibble first)
    q = q.astype(np.uint32).reshape(q.shape[:-1] + (q.shape[-1] // 8, 8))
    w = np.zeros(q.shape[:-1], dtype=np.uint32)
    for i in range(8):
        w |= q[..., i] << np.uint32(4 * i)
    return w.view(np.int32)


def _run_tiny(g):
    lay = _tiny_layer(g)
    gu = MO.gate_up(lay["rows_a"], lay["row_exp"], lay["w1"], lay["s1"], g["I"])
    dc = MO.down_combine(gu["act"], lay["row_tok"], lay["row_w"], lay["row_exp"], lay["w2"], lay["s2"], lay["T"])
    return gu, dc


def test_grouped_gemm_per_expert_zero_points_by_hand():
    # per-group zero points of each expert, element by element in plain Python
    rng = np.random.default_rng(12)
    E, N, K = 2, 3, 256
    q = rng.integers(0, 16, size=(E, N, K)).astype(np.uint8)
    z = rng.integers(6, 10, size=(E, N, K // 128)).astype(np.uint8)
    z[1] = 15 - z[0]                                   # the experts' zero points differ
    s = rng.uniform(0.5, 2.0, size=(E, N, K // 128))
    a = rng.standard_normal((4, K))
    ex = np.array([0, 1, 1, 0])
    got, _ = MO.grouped_gemm(a, ex, _pack(q), s, z)
    for r in range(4):
        e = int(ex[r])
        for n in range(N):
            want = 0.0
            for k in range(K):
                want += float(a[r, k]) * (int(q[e, n, k]) - int(z[e, n, k // 128])) * float(s[e, n, k // 128])
            assert abs(got[r, n] - want) <= 1e-12 * (1 + abs(want))
    # planted: one expert's zero points for every expert
    wrong, _ = MO.grouped_gemm(a, ex, _pack(q), s, np.broadcast_to(z[0], z.shape))
    assert not np.allclose(wrong[ex == 1], got[ex == 1])


def test_moe_tiny_layer_by_hand():
    g = _gold("moe_tiny.json")
    gu, dc = _run_tiny(g)
    T, topk = 2, 2
    gate = gu["g"][:, 0].reshape(T, topk)
    up = gu["u"][:, 0].reshape(T, topk)
    assert np.array_equal(gate, np.array(g["gate"])) and np.array_equal(up, np.array(g["up"]))
    assert np.all(gu["g"][:, 1:] == 0) and np.all(gu["u"][:, 1:] == 0)
    assert np.allclose(gu["act"][:, 0].reshape(T, topk), g["act"], rtol=1e-14, atol=0)
    assert np.allclose(dc["y64"][:, :2], g["y"], rtol=1e-14, atol=1e-16)
    assert np.all(dc["y64"][:, 2:] == 0)


# ------------------------------------------------------ planted mistakes ----

def test_planted_silu_mistakes_fail_the_pins(monkeypatch):
    g = _gold("moe_tiny.json")
    sigmoid = lambda x: 1.0 / (1.0 + np.exp(-x))
    with pytest.raises(AssertionError):
        _check_silu_values(sigmoid)
    # sigmoid in place of SiLU inside the layer changes the hand-worked y
    monkeypatch.setattr(MO, "silu", sigmoid)
    _, dc = _run_tiny(g)
    assert not np.allclose(dc["y64"][:, :2], g["y"], rtol=1e-6)
    monkeypatch.undo()
    # a sign slip in SiLU' fails the finite-difference pin
    def bad_grad(x):
        s = 1.0 / (1.0 + np.exp(-x))
        return s * (1.0 - x * (1.0 - s))
    with pytest.raises(AssertionError):
        _check_silu_grad(bad_grad)
    # ... and makes tau_act miss perturbations
    monkeypatch.setattr(MO, "silu_grad", bad_grad)
    gg, u, tg, tu = _random_gate_up(2000, 5)
    tau = MO.act_bound(gg, u, tg, tu)
    dev = np.abs(MO.silu(gg + tg) * (u + tu) - MO.silu(gg) * u)
    dev = np.maximum(dev, np.abs(MO.silu(gg - tg) * (u - tu) - MO.silu(gg) * u))
    assert np.any(dev > tau)


def test_planted_gate_up_swap_and_dropped_term_fail(monkeypatch):
    g = _gold("moe_tiny.json")
    orig = MO.gate_up

    def swapped(rows_a, row_expert, w1_codes, w1_scales, inter):
        r = orig(rows_a, row_expert, w1_codes, w1_scales, inter)
        act = MO.silu(r["u"]) * r["g"]  # up through SiLU, gate linear
        return dict(r, act=act)
    monkeypatch.setattr(MO, "gate_up", swapped)
    gu, dc = _run_tiny(g)
    assert not np.allclose(gu["act"][:, 0].reshape(2, 2), g["act"], rtol=1e-6)
    monkeypatch.undo()
    # a bound without the Taylor remainder / cross terms misses perturbations
    def first_order_only(gg, u, tg, tu):
        return np.abs(MO.silu_grad(gg) * u) * tg + np.abs(MO.silu(gg)) * tu
    gg, u, tg, tu = _random_gate_up(4000, 11)
    tg, tu = tg * 20, tu * 20  # large boxes make the second-order terms matter
    tau = first_order_only(gg, u, tg, tu)
    dev = np.maximum(np.abs(MO.silu(gg + tg) * (u + tu) - MO.silu(gg) * u),
                     np.abs(MO.silu(gg - tg) * (u - tu) - MO.silu(gg) * u))
    assert np.any(dev > tau)
    assert np.all(dev <= MO.act_bound(gg, u, tg, tu))
