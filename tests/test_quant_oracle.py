"""Pins of the per-token activation quantiser oracle (CPU only).

The oracle (oracle/quant.py) is checked against a hand-worked fixture
(tests/golden/quant_per_token.json), torch's float8_e4m3fn cast, a brute-force
nearest-value search over the code grids, and invariants that hold for any
correct symmetric per-row quantiser.  The last test plants plausible mistakes
in a copy of the rule and checks that these pins reject each one.
"""
import json
import os

import numpy as np
import torch

from oracle import formats as F
from oracle import quant as QZ

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "quant_per_token.json")) as f:
        return json.load(f)


def _rows(seed, m=24, k=200, dtype=torch.bfloat16):
    """fp16/bf16-valued rows with different magnitudes, signs and outliers."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)) * 10.0 ** rng.integers(-3, 4, size=(m, 1))
    x[::5, rng.integers(0, k)] *= -40.0                      # a negative outlier on some rows
    x[3] = 0.0                                               # an all-zero row
    x[4, :] = 0.0
    x[4, 7] = -3.0                                           # a single negative entry
    return torch.from_numpy(x).to(dtype).float().numpy()


def _brute_e4m3(v):
    """Nearest e4m3 code by exhaustive search over the 127 non-negative finite
    codes; ties go to the even code; negative values take the sign bit
    (a value that rounds to zero gives code 0)."""
    vals = F.e4m3_value(np.arange(127))
    out = np.empty(v.shape, dtype=np.uint8)
    for i, x in np.ndenumerate(v):
        d = np.abs(vals - abs(x))
        cand = np.flatnonzero(d == d.min())
        c = int(cand[0]) if len(cand) == 1 else int(cand[cand % 2 == 0][0])
        out[i] = c | 0x80 if (x < 0 and c != 0) else c
    return out


def _brute_int(v):
    """Nearest integer by comparison of floor and floor+1; ties to even."""
    lo = np.floor(v)
    hi = lo + 1
    dlo, dhi = v - lo, hi - v
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return np.clip(pick, -127, 127)


def test_quant_hand_examples():
    g = _gold()
    c, s = QZ.quantize_rows(np.array(g["fp8"]["x"], np.float32), "fp8")
    assert s.tolist() == g["fp8"]["scales"]
    assert c.tolist() == [[int(h, 16) for h in row] for row in g["fp8"]["codes_hex"]]
    c, s = QZ.quantize_rows(np.array(g["int8"]["x"], np.float32), "int8")
    assert s.tolist() == g["int8"]["scales"]
    assert c.tolist() == g["int8"]["codes"]


def test_quant_division_hand_examples():
    # quotients at or next to a rounding tie, where a correctly rounded float32
    # division and a product with a rounded reciprocal give different codes
    g = _gold()
    c, s = QZ.quantize_rows(np.array(g["fp8_division"]["x"], np.float32), "fp8")
    assert s.tolist() == g["fp8_division"]["scales"]
    assert c.tolist() == [[int(h, 16) for h in row] for row in g["fp8_division"]["codes_hex"]]
    c, s = QZ.quantize_rows(np.array(g["int8_division"]["x"], np.float32), "int8")
    assert s.tolist() == g["int8_division"]["scales"]
    assert c.tolist() == g["int8_division"]["codes"]


def test_quant_quotient_against_exact_rationals():
    # the float32 quotient the codes come from is the correctly rounded one:
    # within half a float32 ulp of the exact rational x / s, on every element
    from fractions import Fraction
    x = _rows(21, m=6, k=64)
    for out in ("fp8", "int8"):
        _, s = QZ.quantize_rows(x, out)
        v = (x / s[:, None]).astype(np.float32)
        for (r, c), q in np.ndenumerate(v):
            exact = Fraction(float(x[r, c])) / Fraction(float(s[r]))
            half = Fraction(float(np.spacing(np.float32(abs(q))))) / 2
            assert abs(Fraction(float(q)) - exact) <= half


def test_quant_fp8_codes_match_torch_cast_and_brute_force():
    x = _rows(11)
    codes, s = QZ.quantize_rows(x, "fp8")
    v = (x / s[:, None]).astype(np.float32)                    # the float32 quotient the rule rounds
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    neg_zero = (ref == 0x80)
    assert np.array_equal(codes, np.where(neg_zero, 0, ref))
    sub = v[:6, :40]
    assert np.array_equal(codes[:6, :40], _brute_e4m3(np.clip(sub.astype(np.float64), -448, 448)))


def test_quant_int8_codes_match_brute_force():
    x = _rows(12, dtype=torch.float16)
    codes, s = QZ.quantize_rows(x, "int8")
    v = (x / s[:, None]).astype(np.float32).astype(np.float64)
    assert np.array_equal(codes.astype(np.int64), _brute_int(v).astype(np.int64))


def test_quant_invariants():
    x = _rows(13)
    for out, q in (("fp8", 448.0), ("int8", 127.0)):
        codes, s = QZ.quantize_rows(x, out)
        val = QZ.dequantize_rows(codes, np.ones_like(s), out)
        nz = np.abs(x).max(1) > 0
        # the largest magnitude of a non-zero row lands exactly on +-Q
        assert np.all(np.abs(val[nz]).max(1) == q)
        assert np.all(np.abs(val) <= q)
        # all-zero rows: scale 1, codes 0
        assert np.all(s[~nz] == 1.0) and np.all(val[~nz] == 0)
        # every element within half a code step of x (times s)
        err = np.abs(QZ.dequantize_rows(codes, s, out) - x)
        assert np.all(err <= QZ.step_bound(x, s, out))
        # sign symmetry
        c2, s2 = QZ.quantize_rows(-x, out)
        assert np.array_equal(s2, s)
        assert np.array_equal(QZ.dequantize_rows(c2, s2, out), -QZ.dequantize_rows(codes, s, out))
        # scaling by a power of two moves only the scale (of the non-zero rows)
        c3, s3 = QZ.quantize_rows(x * np.float32(8.0), out)
        assert np.array_equal(c3, codes)
        assert np.array_equal(s3[nz], s[nz] * np.float32(8.0)) and np.all(s3[~nz] == 1.0)


def test_quant_planted_mistakes_are_caught():
    g = _gold()
    xf = np.array(g["fp8"]["x"], np.float32)
    xi = np.array(g["int8"]["x"], np.float32)
    want_f = [[int(h, 16) for h in row] for row in g["fp8"]["codes_hex"]]
    want_i = g["int8"]["codes"]

    def rule(x, out, q=None, absmax=True, rnd=np.rint, recip=False):
        q = np.float32(q if q is not None else (448.0 if out == "fp8" else 127.0))
        m = np.max(np.abs(x) if absmax else x, axis=1)
        s = np.where(m > 0, m / q, np.float32(1)).astype(np.float32)
        den = (x * (np.float32(1) / s)[:, None]) if recip else (x / s[:, None])
        v = np.clip(den.astype(np.float32).astype(np.float64), -float(q), float(q))
        if out == "fp8":
            return F.e4m3_encode(v).tolist()
        return np.clip(rnd(v), -127, 127).astype(np.int64).tolist()

    assert rule(xf, "fp8") == want_f and rule(xi, "int8") == want_i
    assert rule(xi, "int8", q=128.0) != want_i                 # int8 range taken as 128
    assert rule(xi, "int8", rnd=lambda v: np.floor(v + 0.5)) != want_i   # ties away from zero / up
    assert rule(xi, "int8", rnd=np.trunc) != want_i            # truncation
    assert rule(xf, "fp8", q=240.0) != want_f                  # e4m3 "fnuz"-style range
    # quotient as a product with the rounded reciprocal: caught by the division rows
    xd = np.array(g["fp8_division"]["x"], np.float32)
    wd = [[int(h, 16) for h in row] for row in g["fp8_division"]["codes_hex"]]
    assert rule(xd, "fp8") == wd and rule(xd, "fp8", recip=True) != wd
    xdi = np.array(g["int8_division"]["x"], np.float32)
    assert rule(xdi, "int8") == g["int8_division"]["codes"]
    assert rule(xdi, "int8", recip=True) != g["int8_division"]["codes"]
    neg = np.array([[-896, 1, -2, 0.5, 0, 0, 0, 0]], np.float32)
    c, s = QZ.quantize_rows(neg, "fp8")
    assert s.tolist() == [2.0] and rule(neg, "fp8", absmax=False) != c.tolist()   # max without abs


# ------------------------------------------------------------- MXFP4 (W4A4) --

import datagen  # noqa: E402
from oracle import gemm as OG  # noqa: E402


def _mx_fixture():
    with open(os.path.join(GOLD, "mx_w4a4.json")) as f:
        g = json.load(f)
    x = np.zeros((2, 32))
    x[:, :8] = g["x_first8"]
    a = np.zeros((2, 32), np.uint8)
    a[:, :8] = g["a_codes_first8"]
    w = np.zeros((2, 32), np.uint8)
    w[:, :8] = g["w_codes_first8"]
    return g, x, a, w


def test_e2m1_encode_inverts_the_table():
    vals = F.e2m1_value(np.arange(16))
    codes = F.e2m1_encode(vals)
    assert codes.tolist() == [c if c != 8 else 0 for c in range(16)]   # -0 encodes as +0


def test_mx_quantize_hand_example():
    g, x, a, _ = _mx_fixture()
    codes, e8 = QZ.mx_quantize_rows(x)
    assert codes.tolist() == a.tolist()
    assert e8[:, 0].tolist() == g["a_e8m0"]


def _brute_e2m1(v):
    vals = F.e2m1_value(np.arange(8))
    out = np.empty(v.shape, dtype=np.uint8)
    for i, x in np.ndenumerate(v):
        d = np.abs(vals - abs(x))
        cand = np.flatnonzero(d == d.min())
        c = int(cand[0]) if len(cand) == 1 else int(cand[cand % 2 == 0][0])
        out[i] = c | 0x8 if (x < 0 and c != 0) else c
    return out


def test_mx_quantize_brute_force_and_invariants():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((6, 256)) * 10.0 ** rng.integers(-3, 4, size=(6, 1))
    x[2, 64:96] = 0.0                                        # an all-zero block
    x = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    codes, e8 = QZ.mx_quantize_rows(x)
    X = e8.astype(np.int64) - 127
    v = x / np.repeat(np.ldexp(1.0, X), 32, axis=1)
    assert np.array_equal(codes, _brute_e2m1(np.clip(v, -6, 6)))
    mag = np.abs(F.e2m1_value(codes)).reshape(6, 8, 32).max(2)
    nz = np.abs(x).reshape(6, 8, 32).max(2) > 0
    assert np.all(np.isin(mag[nz], (4.0, 6.0))) and np.all(mag[~nz] == 0) and np.all(e8[~nz] == 127)
    c2, e2 = QZ.mx_quantize_rows(-x)
    assert np.array_equal(e2, e8) and np.array_equal(F.e2m1_value(c2), -F.e2m1_value(codes))
    c3, e3 = QZ.mx_quantize_rows(x * 16.0)
    assert np.array_equal(c3, codes) and np.array_equal(e3[nz], e8[nz] + 4)


def test_mx_quantize_planted_mistakes():
    g, x, a, _ = _mx_fixture()

    def rule(emax=2, away=False):
        amax = np.abs(x).max(1, keepdims=True)
        X = np.floor(np.log2(amax)) - emax
        v = np.clip(x / 2.0 ** X, -6, 6)
        if away:  # ties away from zero
            vals = F.e2m1_value(np.arange(8))
            idx = np.array([[np.argmin(np.abs(vals - abs(t)) - 1e-9 * vals) for t in row] for row in v])
            return np.where(v < 0, idx | 8, idx) * (idx != 0)
        return F.e2m1_encode(v)

    assert rule().tolist() == a.tolist()
    assert rule(emax=3).tolist() != a.tolist()
    assert rule(away=True).tolist() != a.tolist()


def test_w4a4_gemm_hand_example_and_integer_special_case():
    g, _, a, w = _mx_fixture()
    r = OG.gemm_mxfp4_mxfp4(datagen.pack_u4(a), np.array(g["a_e8m0"])[:, None], datagen.pack_u4(w),
                            np.array(g["w_e8m0"])[:, None])
    assert r["c64"].tolist() == g["c"]
    # with every scale 2^0, 4 C = (2 e2m1(qa)) . (2 e2m1(qw))^T, an integer matmul
    rng = np.random.default_rng(22)
    qa = rng.integers(0, 16, size=(5, 64), dtype=np.uint8)
    qw = rng.integers(0, 16, size=(7, 64), dtype=np.uint8)
    ia = (2 * F.e2m1_value(qa)).astype(np.int64)
    iw = (2 * F.e2m1_value(qw)).astype(np.int64)
    one = np.full((5, 2), 127)
    r = OG.gemm_mxfp4_mxfp4(datagen.pack_u4(qa), one, datagen.pack_u4(qw), np.full((7, 2), 127))
    assert np.array_equal(r["c64"] * 4, (ia @ iw.T).astype(np.float64))
