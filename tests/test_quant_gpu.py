"""Per-token activation quantiser on the GPU against the oracle, bit for bit.

hq_quantize_per_token decides integer codes from float32 quotients, and the
oracle (oracle/quant.py) takes the same decisions in IEEE float32, so codes
and scales must agree exactly.  Shapes: single rows, rows shorter than one
wave's chunks, ragged lengths, the register-cache boundary (k = 16384) and
rows past it, the W4A8 activation shape (K = 7168, M up to 1024); rows with
zeros, a lone entry, outliers, fp16 extremes and tiny magnitudes.  The last
tests feed the quantiser's output to the W4A8 GEMMs.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_repack_amd as hq
import datagen
from oracle import gemm as og
from oracle import quant as QZ
from oracle.formats import e4m3_value as F_e4m3

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _log(msg):
    print(f"[gpu case] {msg}", flush=True)


def _rows(m, k, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)) * 10.0 ** rng.integers(-2, 3, size=(m, 1))
    if m > 1:
        x[1] = 0.0                                            # all-zero row
    if m > 2:
        x[2] = 0.0
        x[2, k - 1] = -7.5                                    # one entry, at the end of the row
    if m > 3:
        x[3, rng.integers(0, k)] = -3000.0                    # negative outlier
    t = torch.from_numpy(x).to(dtype)
    return t


def _check(x, out):
    codes, scales = hq.quantize_per_token(x.to(DEV), out)
    torch.cuda.synchronize()
    ref_c, ref_s = QZ.quantize_rows(x.float().numpy(), out)
    got_c = codes.cpu().numpy()
    got_s = scales.cpu().numpy()
    bad_s = np.flatnonzero(got_s.view(np.uint32) != ref_s.view(np.uint32))
    assert bad_s.size == 0, f"scales differ in rows {bad_s[:8]}: {got_s[bad_s[:4]]} vs {ref_s[bad_s[:4]]}"
    want = ref_c.view(np.uint8) if out == "int8" else ref_c
    diff = np.argwhere(got_c.view(np.uint8) != want)
    assert diff.size == 0, f"{len(diff)} codes differ, first at {diff[:4].tolist()}"


SHAPES = [(1, 8), (3, 64), (5, 200), (7, 1000), (64, 2048), (17, 7168), (4, 16384), (3, 16392), (2, 40000),
          (1024, 7168)]


@pytest.mark.parametrize("out", ["fp8", "int8"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("m,k", SHAPES)
def test_quantize_matches_oracle_bit_exact(m, k, dt, out):
    _log(f"quantize m={m} k={k} in={dt} out={out}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float16
    _check(_rows(m, k, dtype, seed=m * 31 + k), out)


@pytest.mark.parametrize("out", ["fp8", "int8"])
def test_quantize_extreme_magnitudes(out):
    _log(f"quantize extremes out={out}")
    k = 96
    rows = np.zeros((6, k))
    rows[0, :] = 65504.0 * np.linspace(-1, 1, k)             # fp16 largest finite
    rows[1, :] = 6e-8 * np.arange(k)                          # fp16 subnormals
    rows[2, ::3] = 1.0                                        # ties and exact steps
    rows[3, :] = np.arange(k) - 48.0                          # integers, symmetric
    rows[4, 5] = 2.0 ** -14                                   # one small normal
    rows[5, :] = 1e-4
    _check(torch.from_numpy(rows).to(torch.float16), out)
    tiny = np.random.default_rng(5).standard_normal((4, k)) * np.array([[1e-30], [1e-20], [1e20], [1e30]])
    _check(torch.from_numpy(tiny).to(torch.bfloat16), out)


def _bf16_neighbours(vals, dtype):
    """vals and the next representable values below and above them."""
    t = torch.tensor(vals, dtype=torch.float64).to(dtype)
    bits = t.view(torch.int16).to(torch.int32)
    out = [t]
    for d in (-1, 1):
        out.append((bits + d).to(torch.int16).view(dtype))
    return torch.cat(out)


def test_quantize_every_e4m3_tie():
    """Rows with max 448 (s = 1): every midpoint between neighbouring e4m3
    values, and the values one input step either side, both signs."""
    _log("quantize e4m3 ties")
    vals = F_e4m3(np.arange(127))
    mids = (vals[:-1] + vals[1:]) / 2
    for dtype in (torch.bfloat16, torch.float16):
        pos = _bf16_neighbours(mids[1:], dtype)               # skip the midpoint next to zero's -step
        row = torch.cat([torch.tensor([448.0, 2.0 ** -10], dtype=dtype), pos, -pos])
        row = torch.cat([row, torch.zeros((-row.numel()) % 8, dtype=dtype)])
        _check(row.reshape(1, -1), "fp8")


def test_quantize_every_int8_tie():
    _log("quantize int8 ties")
    halves = np.arange(0, 127) + 0.5
    pos = _bf16_neighbours(halves, torch.float16)
    row = torch.cat([torch.tensor([127.0], dtype=torch.float16), pos, -pos])
    row = torch.cat([row, torch.zeros((-row.numel()) % 8, dtype=torch.float16)])
    _check(row.reshape(1, -1), "int8")


def test_quantize_empty_and_reuse_of_outputs():
    _log("quantize m=0 and preallocated outputs")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    c, s = hq.quantize_per_token(x, "fp8")
    assert c.shape == (0, 64) and s.shape == (0,)
    x = _rows(9, 512, torch.bfloat16, 3)
    codes = torch.full((9, 512), 0x55, dtype=torch.uint8, device=DEV)
    scales = torch.full((9,), -1.0, dtype=torch.float32, device=DEV)
    hq.quantize_per_token(x.to(DEV), "fp8", codes=codes, scales=scales)
    torch.cuda.synchronize()
    ref_c, ref_s = QZ.quantize_rows(x.float().numpy(), "fp8")
    assert np.array_equal(codes.cpu().numpy(), ref_c) and np.array_equal(scales.cpu().numpy(), ref_s)


@pytest.mark.parametrize("M", [1, 16, 128])
def test_quantize_then_w4a8_int_gemm(M):
    N, K = 4096, 7168
    _log(f"quantize -> w4a8-int M={M}")
    x = _rows(M, K, torch.bfloat16, seed=M)
    codes_a, scale_a = hq.quantize_per_token(x.to(DEV), "int8")
    d = datagen.w4a8_int(M, N, K)
    plan = hq.Plan(N, K, hq.w4a8_int(), max_m=M)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
    out = plan.gemm(codes_a, w, meta, a_scale=scale_a)
    torch.cuda.synchronize()
    ref_c, ref_s = QZ.quantize_rows(x.float().numpy(), "int8")
    assert np.array_equal(codes_a.cpu().numpy(), ref_c)
    rows = np.unique(np.linspace(0, M - 1, min(M, 8)).astype(int))
    ref = og.gemm_int4_int8(ref_c[rows], ref_s[rows], d["codes"], d["scales"].double().numpy())
    ok, _, ratio = og.check(out.double().cpu().numpy()[rows], ref["c64"], ref["tau"], "bf16")
    assert ok.all(), f"max err/tau {ratio.max():.3g}"


@pytest.mark.parametrize("M", [1, 16, 128])
def test_quantize_then_w4a8_mxfp4_gemm(M):
    N, K = 4096, 7168
    _log(f"quantize -> w4a8-mxfp4 M={M}")
    x = _rows(M, K, torch.bfloat16, seed=M + 100)
    codes_a, scale_a = hq.quantize_per_token(x.to(DEV), "fp8")
    d = datagen.w4a8_mxfp4(M, N, K)
    plan = hq.Plan(N, K, hq.w4a8_mxfp4(), max_m=M)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    out = plan.gemm(codes_a, w, meta, a_scale=scale_a)
    torch.cuda.synchronize()
    ref_c, ref_s = QZ.quantize_rows(x.float().numpy(), "fp8")
    assert np.array_equal(codes_a.cpu().numpy(), ref_c)
    rows = np.unique(np.linspace(0, M - 1, min(M, 8)).astype(int))
    ref = og.gemm_mxfp4_fp8(ref_c[rows], ref_s[rows], d["codes"], d["e8m0"])
    ok, _, ratio = og.check(out.double().cpu().numpy()[rows], ref["c64"], ref["tau"], "bf16")
    assert ok.all(), f"max err/tau {ratio.max():.3g}"


def test_quantize_honours_timing_events():
    _log("quantize timing events")
    from bench import Hip

    hip = Hip()
    a, b = hip.event(), hip.event()
    x = _rows(128, 7168, torch.bfloat16, 1).to(DEV)
    hq.quantize_per_token(x, "fp8")
    torch.cuda.synchronize()
    hq._check(hq.lib().hq_time_next_launch(a, b))
    hq.quantize_per_token(x, "fp8")
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(a, b)
    hip.destroy(a), hip.destroy(b)
    assert 0.0 < ms < 10.0
