"""Pins of the CPU oracle against things other than itself (CPU only).

Each test pins one part of ``oracle`` to a hand-worked example (tests/golden),
a table typed from a format definition, a library routine (torch's fp8
decoders, numpy's float16 cast, exact integer matmul), exact rational brute
force, or an invariant of the mathematics.  The mutation tests at the end plant
plausible mistakes in the oracle and check that a pin catches each one.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
from oracle import formats as F
from oracle import gemm as G
from oracle import moe as MO

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- unpack ----

def test_unpack_hand_words():
    g = _gold("int4_gemm_2x2.json")
    words = np.array(g["packed_words_int32"], dtype=np.int32).reshape(2, 1)
    assert F.unpack_u4(words).tolist() == g["codes_rows"]
    hexw = np.array([int(h, 16) for h in g["packed_words_hex"]], dtype=np.uint32).view(np.int32)
    assert F.unpack_u4(hexw.reshape(2, 1)).tolist() == g["codes_rows"]


def test_unpack_every_value_every_position():
    for pos in range(8):
        for v in range(16):
            word = np.array([[v << (4 * pos)]], dtype=np.uint32).view(np.int32)
            q = F.unpack_u4(word)[0]
            expect = [0] * 8
            expect[pos] = v
            assert q.tolist() == expect


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(37, 256), dtype=np.uint8)
    assert np.array_equal(F.unpack_u4(datagen.pack_u4(q)), q)
    words = rng.integers(-2**31, 2**31, size=(5, 9), dtype=np.int64).astype(np.int32)
    assert np.array_equal(datagen.pack_u4(F.unpack_u4(words)), words)


# ---------------------------------------------------------- code tables ----

def test_e2m1_table_from_definition():
    vals = F.e2m1_value(np.arange(16))
    expect = np.array(_gold("e2m1_table.json")["values"])
    assert np.array_equal(vals, expect)
    assert np.array_equal(np.signbit(vals), np.signbit(expect))


def test_e8m0_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    ours = F.e8m0_value(np.arange(256))
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def test_e4m3_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = F.e4m3_value(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_int8_value():
    assert F.int8_value(np.array([0, 1, 127, 128, 255], dtype=np.uint8)).tolist() == [0, 1, 127, -128, -1]


# ------------------------------------------------------------- rounding ----

def test_rne_f16_matches_numpy_cast():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, size=20000),
        np.array([2.0 ** -24 * 1.5, 2.0 ** -24 * 2.5, 2.0 ** -14, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11]),
    ])
    x = x[np.abs(x) < 65000]
    assert np.array_equal(F.rne(x, "f16"), x.astype(np.float16).astype(np.float64))


def test_rne_bf16_matches_torch_cast_on_fp32_inputs():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, size=20000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(F.rne(x.astype(np.float64), "bf16"), ref)


def test_rne_e4m3_and_encode_match_torch_cast():
    rng = np.random.default_rng(4)
    x = np.clip(rng.standard_normal(20000) * 10.0 ** rng.integers(-4, 3, size=20000), -448, 448)
    x = x.astype(np.float32)
    ref_codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref_vals = F.e4m3_value(ref_codes)
    assert np.array_equal(F.rne(x.astype(np.float64), "e4m3"), ref_vals)
    ours = F.e4m3_encode(x.astype(np.float64))
    same = (ours == ref_codes) | ((ours & 0x7F) == 0) & ((ref_codes & 0x7F) == 0)
    assert same.all()


# ------------------------------------------------------------ dequant ----

def test_dequant_int4_brute_force_rational():
    scales16 = [0.005, 0.0123, 0.02, 1.0, 0.33]
    for dt in (torch.float16, torch.bfloat16):
        svals = torch.tensor(scales16, dtype=torch.float32).to(dt).double().numpy()
        for s in svals:
            for z in range(16):
                q = np.arange(16, dtype=np.uint8)
                codes = datagen.pack_u4(np.tile(q, (1, 8))[:, :128])
                w = G.dequant_int4(codes, np.array([[s]]), np.array([[z]]), group=128)[0, :16]
                expect = [Fraction(int(c) - z) * Fraction(float(s)) for c in q]
                assert [Fraction(float(v)) for v in w] == expect


def test_dequant_group_mapping():
    # zero point of group g must only affect k in [128 g, 128 g + 128)
    q = np.full((1, 512), 8, dtype=np.uint8)
    codes = datagen.pack_u4(q)
    zeros = np.array([[8, 9, 8, 7]])
    w = G.dequant_int4(codes, np.ones((1, 4)), zeros, 128)[0]
    assert np.all(w[:128] == 0) and np.all(w[128:256] == -1) and np.all(w[256:384] == 0)
    assert np.all(w[384:] == 1)


# ---------------------------------------------------- hand GEMM examples ----

def test_int4_gemm_hand_example():
    g = _gold("int4_gemm_2x2.json")
    codes = datagen.pack_u4(np.array(g["codes_rows"], dtype=np.uint8))
    r = G.gemm_w4a16(np.array(g["a"], float), codes, np.array(g["scales"]), g["zero"], group=g["group"])
    assert r["c64"].tolist() == g["c"]
    assert r["c_out"].tolist() == g["c"]


def test_int4_int8_accumulators_hand_example():
    g = _gold("int4_gemm_2x2.json")
    codes = datagen.pack_u4(np.array(g["codes_rows"], dtype=np.uint8))
    a = np.array(g["a"], dtype=np.int64).astype(np.int8)
    r = G.gemm_int4_int8(a, np.ones(2, np.float32), codes, np.array(g["scales"]), group=g["group"])
    assert r["P"].tolist() == g["int_accumulators_P"]
    assert r["c64"].tolist() == g["c"]


def test_mxfp4_gemm_hand_example():
    g = _gold("mxfp4_gemm_2x2.json")
    q = np.zeros((2, 32), dtype=np.uint8)
    q[:, :2] = np.array(g["w_codes_rows_first_two"])
    assert F.e2m1_value(q[:, :2]).tolist() == g["w_values_first_two"]
    a = np.full((2, 32), g["a_rest"])
    a[:, :2] = np.array(g["a_first_two"])
    a_codes = F.e4m3_encode(a)
    assert np.array_equal(F.e4m3_value(a_codes), a)
    r = G.gemm_mxfp4_fp8(a_codes, np.array(g["a_scale"], np.float32), datagen.pack_u4(q),
                         np.array(g["e8m0"], np.uint8).reshape(2, 1))
    assert r["c64"].tolist() == g["c"]


# ------------------------------------------------- general GEMM pins ----

def test_integer_weight_special_case_equals_int_matmul():
    rng = np.random.default_rng(5)
    M, N, K = 7, 9, 256
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    a = rng.integers(-50, 50, size=(M, K)).astype(np.float64)
    r = G.gemm_w4a16(a, datagen.pack_u4(q), np.ones((N, K // 128)), 0)
    assert np.array_equal(r["c64"], (a.astype(np.int64) @ q.astype(np.int64).T).astype(np.float64))


def test_exact_rational_brute_force_small():
    rng = np.random.default_rng(6)
    for M, N, K in [(1, 1, 128), (3, 2, 256), (2, 3, 128)]:
        d = datagen.dense_w4a16(M, N, K, act="f16", zp="u4", key=(99,))
        a = d["a"].double().numpy()
        s = d["scales"].double().numpy()
        q = F.unpack_u4(d["codes"])
        r = G.gemm_w4a16(a, d["codes"], s, d["zeros"])
        for m in range(M):
            for n in range(N):
                exact = sum(Fraction(float(a[m, k])) * (int(q[n, k]) - int(d["zeros"][n, k // 128]))
                            * Fraction(float(s[n, k // 128])) for k in range(K))
                err = abs(Fraction(float(r["c64"][m, n])) - exact)
                assert err <= Fraction(2.0 ** -40) * (1 + abs(exact))


def test_mxfp4_inner_sum_exact_against_rational():
    d = datagen.w4a8_mxfp4(2, 3, 256, key=(98,))
    r = G.gemm_mxfp4_fp8(d["a_codes"].numpy(), np.ones(2, np.float32), d["codes"], d["e8m0"])
    a = F.e4m3_value(d["a_codes"].numpy())
    q = F.unpack_u4(d["codes"])
    for m in range(2):
        for n in range(3):
            exact = sum(Fraction(float(a[m, k])) * Fraction(float(F.e2m1_value(q[n, k])))
                        * Fraction(2) ** (int(d["e8m0"][n, k // 32]) - 127) for k in range(256))
            assert Fraction(float(r["c64"][m, n])) == exact


def test_invariants():
    d = datagen.dense_w4a16(5, 6, 384, act="bf16", zp="u4", key=(97,))
    a = d["a"].double().numpy()
    s = d["scales"].double().numpy()
    base = G.gemm_w4a16(a, d["codes"], s, d["zeros"])["c64"]
    # scales x2 -> C exactly x2
    assert np.array_equal(G.gemm_w4a16(a, d["codes"], 2 * s, d["zeros"])["c64"], 2 * base)
    # shifting codes and zero points of a group by the same delta leaves C unchanged
    q = F.unpack_u4(d["codes"]).astype(np.int64)
    q[:, 128:256] = np.maximum(q[:, 128:256], 3)
    z = d["zeros"].astype(np.int64)
    c1 = G.gemm_w4a16(a, datagen.pack_u4(q.astype(np.uint8)), s, z)["c64"]
    q2 = q.copy()
    q2[:, 128:256] -= 3
    z2 = z.copy()
    z2[:, 1] -= 3
    assert q2.min() >= 0
    c2 = G.gemm_w4a16(a, datagen.pack_u4(q2.astype(np.uint8)), s, z2)["c64"]
    assert np.allclose(c2, c1, rtol=0, atol=1e-12)
    # permuting A's rows permutes C's rows
    perm = np.array([3, 0, 4, 1, 2])
    assert np.array_equal(G.gemm_w4a16(a[perm], d["codes"], s, d["zeros"])["c64"], base[perm])


def test_mxfp4_scale_exponent_invariant():
    d = datagen.w4a8_mxfp4(3, 4, 128, key=(96,))
    ac, sa = d["a_codes"].numpy(), d["a_scale"].numpy()
    base = G.gemm_mxfp4_fp8(ac, sa, d["codes"], d["e8m0"])["c64"]
    e2 = d["e8m0"].copy()
    e2[:, 2] += 1  # block 2 (k in [64, 96)) contribution doubles
    c2 = G.gemm_mxfp4_fp8(ac, sa, d["codes"], e2)["c64"]
    only = d["e8m0"].copy()
    only_codes = F.unpack_u4(d["codes"]).copy()
    only_codes[:, :64] = 0
    only_codes[:, 96:] = 0
    blk = G.gemm_mxfp4_fp8(ac, sa, datagen.pack_u4(only_codes), only)["c64"]
    assert np.allclose(c2 - base, blk, rtol=1e-14, atol=1e-14)


def test_int_accumulators_against_loops():
    d = datagen.w4a8_int(3, 2, 256, key=(95,))
    P = G.int_accumulators(d["a_codes"].numpy(), d["codes"])
    a = d["a_codes"].numpy().astype(np.int64)
    q = F.unpack_u4(d["codes"]).astype(np.int64)
    for m in range(3):
        for n in range(2):
            for g in range(2):
                assert P[m, n, g] == sum(int(a[m, k]) * (int(q[n, k]) - 8) for k in range(128 * g, 128 * g + 128))


def test_tolerance_rule_accepts_exact_rounding():
    for act in ("f16", "bf16"):
        d = datagen.dense_w4a16(16, 64, 1024, act=act, zp="u4", key=(94,))
        r = G.gemm_w4a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), d["zeros"],
                         out_fmt=act)
        ok, _, _ = G.check(r["c_out"], r["c64"], r["tau"], act)
        assert ok.all()
        # a result off by 3 tau is rejected
        bad, _, _ = G.check(r["c64"] + 3 * r["tau"] + 1e-3, r["c64"], r["tau"], act)
        assert not bad.any()


# ----------------------------------------------------------------- MoE ----

def _small_moe(T=6, E=4, topk=2, H=256, I=128, act="bf16", key=(93,)):
    rt = datagen.moe_routing(T, E, topk, key=key)
    w = datagen.moe_weights(E, H, I, key=key)
    x = datagen.moe_activations(T, H, act, key=key)
    return rt, w, x


def test_moe_single_expert_reduces_to_dense():
    T, H, I = 5, 256, 128
    _, w, x = _small_moe(T=T, E=1, topk=1, H=H, I=I)
    xa = x["x"].double().numpy()
    s1 = w["s1"].double().numpy()
    s2 = w["s2"].double().numpy()
    ids = np.zeros((T, 1), np.int32)
    gu = MO.gate_up(xa, ids.reshape(-1), w["w1"], s1, I)
    h = G.gemm_w4a16(xa, w["w1"][0], s1[0], 8)["c64"]
    assert np.array_equal(gu["g"], h[:, :I]) and np.array_equal(gu["u"], h[:, I:])
    act = F.rne(gu["act"], "bf16")
    dc = MO.down_combine(act, np.arange(T), np.ones(T), np.zeros(T, int), w["w2"], s2, T)
    o = G.gemm_w4a16(act, w["w2"][0], s2[0], 8)["c64"]
    assert np.array_equal(dc["y64"], o)


def test_moe_combine_matches_per_token_loop():
    T, E, topk, H, I = 4, 3, 2, 256, 128
    rt, w, x = _small_moe(T, E, topk, H, I)
    xa = x["x"].double().numpy()
    ids, tw = rt["topk_ids"], rt["topk_w"]
    s1, s2 = w["s1"].double().numpy(), w["s2"].double().numpy()
    rows = np.repeat(xa, topk, axis=0)
    gu = MO.gate_up(rows, ids.reshape(-1), w["w1"], s1, I)
    dc = MO.down_combine(gu["act"], np.repeat(np.arange(T), topk), tw.reshape(-1), ids.reshape(-1),
                         w["w2"], s2, T)
    for t in range(T):
        y = np.zeros(H)
        for j in range(topk):
            e = ids[t, j]
            W1 = G.dequant_int4(w["w1"][e], s1[e], 8)
            W2 = G.dequant_int4(w["w2"][e], s2[e], 8)
            h = W1 @ xa[t]
            a = h[:I] / (1 + np.exp(-h[:I])) * h[I:]
            y += float(tw[t, j]) * (W2 @ a)
        assert np.allclose(dc["y64"][t], y, rtol=1e-12, atol=1e-12)


def _align_ref(ids, E, bm):
    flat = ids.reshape(-1)
    sid, bexp = [], []
    for e in range(E + 1):  # the experts, then the out-of-range ids
        sel = (flat == e) if e < E else ((flat < 0) | (flat >= E))
        rows = list(np.nonzero(sel)[0])
        nb = -(-len(rows) // bm)
        rows += [flat.size] * (nb * bm - len(rows))
        sid += rows
        bexp += [e if e < E else -1] * nb
    return np.array(sid), np.array(bexp), np.array([len(sid)])


def test_align_out_of_range_ids_form_the_last_segment():
    ids = np.array([[0, -1], [3, 4], [2, 0], [-1, 7], [1, 1]])  # E = 4: -1, 4 and 7 are out of range
    sid, bexp, npad = _align_ref(ids, 4, 2)
    assert MO.check_align(ids, 4, 2, sid, bexp, npad)
    assert list(bexp[-2:]) == [-1, -1] and sorted(sid[-4:]) == [1, 3, 6, 7]
    be = bexp.copy()
    be[-1] = 3  # the out-of-range block labelled as an expert
    with pytest.raises(AssertionError):
        MO.check_align(ids, 4, 2, sid, be, npad)
    # dropping the out-of-range segment is not a valid alignment
    with pytest.raises(AssertionError):
        MO.check_align(ids, 4, 2, sid[:-4], bexp[:-2], npad - 4)


def test_align_invariants_accept_and_reject():
    rt, _, _ = _small_moe(T=9, E=4, topk=2)
    ids = rt["topk_ids"]
    sid, bexp, npad = _align_ref(ids, 4, 4)
    assert MO.check_align(ids, 4, 4, sid, bexp, npad)
    # reorder inside a segment: still valid
    s2 = sid.copy()
    s2[:2] = s2[:2][::-1]
    assert MO.check_align(ids, 4, 4, s2, bexp, npad)
    bad = sid.copy()
    bad[0] = bad[1]  # duplicate slot
    with pytest.raises(AssertionError):
        MO.check_align(ids, 4, 4, bad, bexp, npad)
    be = bexp.copy()
    be[0] = (be[0] + 1) % 4
    with pytest.raises(AssertionError):
        MO.check_align(ids, 4, 4, sid, be, npad)
    with pytest.raises(AssertionError):
        MO.check_align(ids, 4, 4, np.concatenate([sid, [18] * 4]), np.concatenate([bexp, [3]]), npad + 4)


def test_requant_fp8_rows_definition():
    rng = np.random.default_rng(7)
    act = rng.standard_normal((5, 256)) * 3
    dq, s = MO.requant_fp8_rows(act)
    assert np.allclose(s, np.abs(act).max(1) / 448.0)
    assert np.all(np.abs(dq - act) <= 0.5 * F.ulp(np.abs(act) / s[:, None], "e4m3") * s[:, None] * (1 + 1e-12))
    zero_dq, zero_s = MO.requant_fp8_rows(np.zeros((1, 8)))
    assert zero_s[0] == 1.0 and np.all(zero_dq == 0)


def test_routing_matches_full_sort():
    rt = datagen.moe_routing(16, 256, 8, key=(92,))
    rng = datagen.rng_for(92, 16, 256, 8, 1)
    logits = rng.standard_normal((16, 256))
    for t in range(16):
        p = np.exp(logits[t] - logits[t].max())
        p /= p.sum()
        order = sorted(range(256), key=lambda e: (-p[e], e))[:8]
        assert rt["topk_ids"][t].tolist() == order
        assert np.allclose(rt["topk_w"][t], p[order].astype(np.float32))


# ------------------------------------------- planted mistakes are caught ----

def test_planted_mistakes_are_caught(monkeypatch):
    g = _gold("int4_gemm_2x2.json")
    codes = datagen.pack_u4(np.array(g["codes_rows"], dtype=np.uint8))
    a = np.array(g["a"], float)

    def run():
        return G.gemm_w4a16(a, codes, np.array(g["scales"]), g["zero"], group=g["group"])["c64"].tolist()

    assert run() == g["c"]
    # high-nibble-first unpack
    def bad_unpack(words):
        w = np.ascontiguousarray(words).view(np.uint32)
        out = np.empty(w.shape[:-1] + (w.shape[-1] * 8,), dtype=np.uint8)
        for i in range(8):
            out[..., i::8] = (w >> np.uint32(28 - 4 * i)) & np.uint32(0xF)
        return out
    monkeypatch.setattr(G, "unpack_u4", bad_unpack)
    assert run() != g["c"]
    monkeypatch.undo()
    # zero point added instead of subtracted: w = (q + z) * s
    def bad_dequant(c, s, z, group=128):
        q = F.unpack_u4(c).astype(np.float64)
        return (q + float(z)) * np.repeat(np.asarray(s, float), group, axis=1)
    monkeypatch.setattr(G, "dequant_int4", bad_dequant)
    assert run() != g["c"]
    monkeypatch.undo()
    # scale taken from the wrong group index (k // 8 instead of k // group)
    def bad_group(c, s, z, group=128):
        q = F.unpack_u4(c).astype(np.float64)
        sc = np.asarray(s, float)
        idx = np.minimum(np.arange(q.shape[1]) // 1, sc.shape[1] - 1)
        return (q - float(z)) * sc[:, idx] * np.where(np.arange(q.shape[1]) % 2, 0.5, 1.0)
    monkeypatch.setattr(G, "dequant_int4", bad_group)
    assert run() != g["c"]
    monkeypatch.undo()
    # transposed weight operand (C = A W rather than A W^T) cannot even be formed
    # for non-square shapes; the 2x2 example catches a swapped output instead:
    assert np.array(run()).T.tolist() != g["c"]
    # a wrong E2M1 exponent bias is caught by the table pin
    vals = F.e2m1_value(np.arange(16)) * 2
    assert not np.array_equal(vals, np.array(_gold("e2m1_table.json")["values"]))


# ------------------------------------------------------------ INT8 weights --

def test_int8_gemm_hand_example():
    g = _gold("int8_gemm_2x2.json")
    r = G.gemm_w8a16(np.array(g["a"], float), np.array(g["codes"], np.uint8), np.array(g["scales"]), g["zero"],
                     group=g["group"])
    assert r["c64"].tolist() == g["c"]
    # the same bytes given as int32 words (low byte first)
    words = np.array(g["codes"], np.uint8).view(np.int32)
    assert np.array_equal(G.dequant_int8(words, np.array(g["scales"]), g["zero"], group=8),
                          G.dequant_int8(np.array(g["codes"], np.uint8), np.array(g["scales"]), g["zero"], group=8))


def test_int8_weights_agree_with_int4_on_shared_range():
    """Codes 120..135 with zero 128 are the INT4 codes 0..15 with zero 8."""
    rng = np.random.default_rng(31)
    q4 = rng.integers(0, 16, size=(6, 256), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, size=(6, 2))
    w4 = G.dequant_int4(datagen.pack_u4(q4), s, 8)
    w8 = G.dequant_int8((q4.astype(np.int64) + 120).astype(np.uint8), s, 128)
    assert np.array_equal(w4, w8)


def test_int8_integer_special_case():
    rng = np.random.default_rng(32)
    q = rng.integers(0, 256, size=(7, 384), dtype=np.uint8)
    a = rng.integers(-4, 5, size=(5, 384)).astype(np.float64)
    r = G.gemm_w8a16(a, q, np.ones((7, 3)), 128)
    ref = a.astype(np.int64) @ (q.astype(np.int64) - 128).T
    assert np.array_equal(r["c64"], ref.astype(np.float64))


# ------------------------------------------------------------ INT2 weights --

def test_int2_unpack_and_gemm_hand_example():
    g = _gold("int2_gemm_2x2.json")
    words = np.array([int(h, 16) for h in g["packed_words_hex"]], dtype=np.uint32).view(np.int32).reshape(2, 1)
    assert G.unpack_u2(words).tolist() == g["codes_rows"]
    r = G.gemm_w2a16(np.array(g["a"], float), words, np.array(g["scales"]), g["zero"], group=g["group"])
    assert r["c64"].tolist() == g["c"]


def test_int2_unpack_every_value_every_position():
    for pos in range(16):
        for v in range(4):
            word = np.array([[v << (2 * pos)]], dtype=np.uint32).view(np.int32)
            q = G.unpack_u2(word)[0]
            expect = [0] * 16
            expect[pos] = v
            assert q.tolist() == expect


def test_int2_weights_agree_with_int4_on_shared_range():
    """Codes 0..3 with zero 2 are the INT4 codes 6..9 with zero 8."""
    rng = np.random.default_rng(33)
    q2 = rng.integers(0, 4, size=(5, 256), dtype=np.uint8)
    words = np.zeros((5, 16), np.uint32)
    for i in range(16):
        words |= (q2[:, i::16].astype(np.uint32) << np.uint32(2 * i))
    s = rng.uniform(0.005, 0.02, size=(5, 2))
    w2 = G.dequant_int2(words.view(np.int32), s, 2)
    w4 = G.dequant_int4(datagen.pack_u4(q2 + 6), s, 8)
    assert np.array_equal(w2, w4)


# ------------------------------------------------------------ INT3 weights --

def test_int3_unpack_and_gemm_hand_example():
    g = _gold("int3_gemm_2x2.json")
    words = np.array([[int(h, 16) for h in row] for row in g["packed_words_hex"]], dtype=np.uint32).view(np.int32)
    assert G.unpack_u3(words).tolist() == g["codes_rows"]
    r = G.gemm_w3a16(np.array(g["a"], float), words, np.array(g["scales"]), g["zero"], group=g["group"])
    assert r["c64"].tolist() == g["c"]


def _stream_words(rows):
    """Test-side packer: each row of 3-bit codes as one Python integer bit
    stream, cut into 32-bit words (lowest first)."""
    out = []
    for codes in rows:
        v = 0
        for k, q in enumerate(codes):
            v |= int(q) << (3 * k)
        out.append([(v >> (32 * j)) & 0xFFFFFFFF for j in range(len(codes) * 3 // 32)])
    return np.array(out, dtype=np.uint32).view(np.int32)


def test_int3_unpack_every_value_every_position():
    """Each of the 8 values at each of the 32 positions of a 3-word group,
    including the straddling positions 10 and 21."""
    for pos in range(32):
        for v in range(8):
            words = np.array([[((v << (3 * pos)) >> (32 * j)) & 0xFFFFFFFF for j in range(3)]],
                             dtype=np.uint32).view(np.int32)
            q = G.unpack_u3(words)[0]
            expect = [0] * 32
            expect[pos] = v
            assert q.tolist() == expect


def test_int3_weights_agree_with_int4_on_shared_range():
    """Codes 0..7 with zero 4 are the INT4 codes 4..11 with zero 8."""
    rng = np.random.default_rng(34)
    q3 = rng.integers(0, 8, size=(5, 256), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, size=(5, 2))
    w3 = G.dequant_int3(_stream_words(q3), s, 4)
    w4 = G.dequant_int4(datagen.pack_u4(q3 + 4), s, 8)
    assert np.array_equal(w3, w4)


# ---------------------------------------------------------- MXINT4 weights --

def test_mxint4_hand_example():
    g = _gold("mxint4_gemm_2x2.json")
    words = np.array([[int(h, 16) for h in row] for row in g["packed_words_hex"]], dtype=np.uint32).view(np.int32)
    assert F.unpack_u4(words).tolist() == g["codes_rows"]
    r = G.gemm_mxint4_w16(np.array(g["a"], float), words, np.array(g["e8m0"], dtype=np.uint8))
    assert r["c64"].tolist() == g["c"]


def test_mxint4_every_code():
    """The 16 codes are the two's-complement integers -8..7 in quarters."""
    vals = F.mxint4_value(np.arange(16))
    assert vals.tolist() == [0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, -2, -1.75, -1.5, -1.25, -1, -0.75, -0.5, -0.25]


def test_mxint4_weights_agree_with_int4_group32():
    """A two's-complement code q is the INT4 code q xor 8 with zero 8; the
    implicit 2^-2 and the E8M0 block scale make a group-32 scale 2^(X-129)."""
    rng = np.random.default_rng(35)
    q = rng.integers(0, 16, size=(6, 256), dtype=np.uint8)
    x = rng.integers(100, 140, size=(6, 8))
    w_mx = G.mxint4_weights(datagen.pack_u4(q), x.astype(np.uint8))
    w_i4 = G.dequant_int4(datagen.pack_u4(q ^ 8), np.ldexp(1.0, x - 129), 8, group=32)
    assert np.array_equal(w_mx, w_i4)


def test_mxint4_nan_scale_propagates():
    q = np.zeros((1, 32), np.uint8)
    q[0, 3] = 5
    w = G.mxint4_weights(datagen.pack_u4(q), np.array([[255]], np.uint8))
    assert np.isnan(w).all()


# ----------------------------------------------------------- NVFP4 weights --

def test_nvfp4_hand_example():
    g = _gold("nvfp4_gemm_2x2.json")
    words = np.array([[int(h, 16) for h in row] for row in g["packed_words_hex"]], dtype=np.uint32).view(np.int32)
    assert F.unpack_u4(words).tolist() == g["codes_rows"]
    r = G.gemm_nvfp4_w16(np.array(g["a"], float), words, np.array(g["e4m3_scales"], dtype=np.uint8),
                         g["tensor_scale"])
    assert r["c64"].tolist() == g["c"]


def test_nvfp4_agrees_with_mxfp4_on_power_of_two_scales():
    """E4M3 scales that are powers of two, equal on both halves of every 32-block,
    with tensor scale 1, are E8M0 block scales: the MXFP4 weights."""
    rng = np.random.default_rng(36)
    q = rng.integers(0, 16, size=(5, 256), dtype=np.uint8)
    ex = rng.integers(-6, 8, size=(5, 8))            # 2^ex, all E4M3 normals
    e4 = ((ex + 7) << 3).astype(np.uint8)            # E4M3 code of 2^ex (mantissa 0)
    w_nv = G.nvfp4_weights(datagen.pack_u4(q), np.repeat(e4, 2, axis=1), 1.0)
    w_mx = G.mxfp4_weights(datagen.pack_u4(q), (ex + 127).astype(np.uint8))
    assert np.array_equal(w_nv, w_mx)


def test_nvfp4_block_of_16_and_tensor_scale():
    """Each 16-block takes its own scale, and the tensor scale multiplies all."""
    q = np.full((1, 32), 0x2, np.uint8)              # E2M1 1.0 everywhere
    w = G.nvfp4_weights(datagen.pack_u4(q), np.array([[0x38, 0x40]], np.uint8), 0.5)
    assert w[0, :16].tolist() == [0.5] * 16 and w[0, 16:].tolist() == [1.0] * 16
    wn = G.nvfp4_weights(datagen.pack_u4(q), np.array([[0x7F, 0x40]], np.uint8), 1.0)
    assert np.isnan(wn[0, :16]).all() and (wn[0, 16:] == 2.0).all()
