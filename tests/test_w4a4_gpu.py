"""W4A4 (MXFP4 activations x MXFP4 weights) on the GPU against the oracle.

The GEMM outputs must lie within the oracle's tolerance (tau + half an output
ulp, oracle/gemm.py) on both kernels and the automatic choice, over the
W4A8 layer shape (N = 4096, K = 7168) at M in {1, 16, 128, 1024} (sampled
rows for the large M) and ragged shapes that span several tiles.  The MXFP4
activation quantiser must match the oracle bit for bit, and its output fed to
the GEMM must give the oracle's result.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_repack_amd as hq
import datagen
from oracle import gemm as og
from oracle import quant as QZ

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _log(msg):
    print(f"[gpu case] {msg}", flush=True)


def _rows(M):
    return np.unique(np.linspace(0, M - 1, min(M, 12)).astype(int))


def _run(M, N, K, tuning=None):
    _log(f"w4a4 M={M} N={N} K={K} tuning={tuning}")
    d = datagen.w4a4_mxfp4(M, N, K)
    plan = hq.Plan(N, K, hq.w4a4_mxfp4(), max_m=M, tuning=tuning)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    a = torch.from_numpy(d["a_codes"]).to(DEV)
    ea = hq.mx_scales_group_major(torch.from_numpy(d["a_e8m0"])).to(DEV)
    out = plan.gemm(a, w, meta, a_scale=ea)
    torch.cuda.synchronize()
    rows = _rows(M)
    ref = og.gemm_mxfp4_mxfp4(d["a_codes"][rows], d["a_e8m0"][rows], d["codes"], d["e8m0"])
    ok, _, ratio = og.check(out.double().cpu().numpy()[rows], ref["c64"], ref["tau"], "bf16")
    assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"
    return plan.describe(M)


@pytest.mark.parametrize("kernel", [0, 1, 2])
@pytest.mark.parametrize("M", [1, 16, 128, 1024])
def test_w4a4_layer_shape(M, kernel):
    _run(M, 4096, 7168, None if kernel == 0 else dict(kernel=kernel))


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (3, 256, 256), (37, 384, 640), (70, 512, 1152), (200, 256, 384)])
def test_w4a4_ragged(M, N, K):
    _run(M, N, K)
    _run(M, N, K, dict(kernel=1, tile_m=16 * (1 if M <= 16 else 2), tile_n=32))


@pytest.mark.parametrize("tuning", [dict(kernel=2, tile_m=64, tile_n=128, stages=2),
                                    dict(kernel=2, tile_m=128, tile_n=256, stages=5),
                                    dict(kernel=2, tile_m=64, tile_n=128, split_k=3),
                                    dict(kernel=1, split_k=4)])
def test_w4a4_tunings(tuning):
    _run(96, 512, 1536, tuning)


def _mx_check(x):
    codes, e8 = hq.quantize_mxfp4(x.to(DEV))
    torch.cuda.synchronize()
    ref_c, ref_e = QZ.mx_quantize_rows(x.float().numpy())
    got = codes.cpu().numpy()
    want = (ref_c[:, 0::2] | (ref_c[:, 1::2] << 4)).astype(np.uint8)
    m = ref_e.shape[0]
    ref_words = ref_e.reshape(m, -1, 4).transpose(1, 0, 2)   # the group-major word layout
    assert np.array_equal(e8.cpu().numpy(), ref_words), "E8M0 scales differ"
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:4].tolist()}"
    return codes, e8


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("m,k", [(1, 128), (3, 384), (17, 7168), (256, 4096), (1024, 7168)])
def test_quantize_mxfp4_bit_exact(m, k, dt):
    _log(f"quantize mxfp4 m={m} k={k} {dt}")
    rng = np.random.default_rng(m * 7 + k)
    x = rng.standard_normal((m, k)) * 10.0 ** rng.integers(-3, 4, size=(m, 1))
    if m > 2:
        x[1, :32] = 0.0                                       # an all-zero block
        x[2, 40] = -5000.0 if dt == torch.float16 else -5e9    # an outlier block
    _mx_check(torch.from_numpy(x).to(dt))


def test_quantize_mxfp4_ties_and_extremes():
    _log("quantize mxfp4 ties and extremes")
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mids = (e2m1[:-1] + e2m1[1:]) / 2
    blk = np.zeros(32)
    blk[0] = 6.0                                              # X = 0
    blk[1:8] = mids
    blk[8:15] = -mids
    blk[15:22] = mids * 1.0078125                              # just above each midpoint
    x = np.concatenate([blk, blk * 2.0 ** -20, blk * 2.0 ** 20, np.r_[blk[:16], 7.5, 6.5, np.zeros(14)]])
    _mx_check(torch.from_numpy(x[None, :]).to(torch.bfloat16))
    tiny = np.zeros((1, 128))
    tiny[0, :4] = [1e-38, -2e-39, 3e-40, 0]                   # subnormal block maximum
    _mx_check(torch.from_numpy(tiny).to(torch.bfloat16))


@pytest.mark.parametrize("M", [1, 16, 128])
def test_quantize_mxfp4_then_w4a4_gemm(M):
    N, K = 4096, 7168
    _log(f"quantize mxfp4 -> w4a4 M={M}")
    x = torch.from_numpy(np.random.default_rng(M).standard_normal((M, K))).to(torch.bfloat16)
    codes, e8 = _mx_check(x)
    d = datagen.w4a4_mxfp4(M, N, K)
    plan = hq.Plan(N, K, hq.w4a4_mxfp4(), max_m=M)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    out = plan.gemm(codes, w, meta, a_scale=e8)
    torch.cuda.synchronize()
    ref_c, ref_e = QZ.mx_quantize_rows(x.float().numpy())
    rows = _rows(M)
    ref = og.gemm_mxfp4_mxfp4(datagen.pack_u4(ref_c[rows]), ref_e[rows], d["codes"], d["e8m0"])
    ok, _, ratio = og.check(out.double().cpu().numpy()[rows], ref["c64"], ref["tau"], "bf16")
    assert ok.all(), f"max err/tau {ratio.max():.3g}"
