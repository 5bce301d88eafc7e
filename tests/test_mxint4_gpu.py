"""W4A16-MXINT4 (MXINT4 weights, fp16 / bf16 activations) on the GPU against
the oracle.

Every output must lie within the oracle's tolerance (tau + half an output ulp,
oracle/gemm.py) on both kernels and the automatic choice, over decode and
prefill-sized M at N = K = 4096 (sampled rows for the large M), ragged shapes
spanning several tiles and the tile tunings; an E8M0 code 255 (NaN) makes
exactly the outputs of its column NaN; the GPU repack equals the host repack
byte for byte.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_repack_amd as hq
import datagen
from oracle import gemm as og

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _log(msg):
    print(f"[gpu case] {msg}", flush=True)


def _run(M, N, K, act, tuning=None, d=None):
    _log(f"w4a16-mxint4 M={M} N={N} K={K} act={act} tuning={tuning}")
    d = d or datagen.w4a16_mxint4(M, N, K, act=act)
    plan = hq.Plan(N, K, hq.w4a16_mxint4(act), max_m=M, tuning=tuning)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    out = plan.gemm(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, min(M, 12)).astype(int))
    ref = og.gemm_mxint4_w16(d["a"].double().numpy()[rows], d["codes"], d["e8m0"], out_fmt=act)
    got = out.double().cpu().numpy()[rows]
    return got, ref


def _check(got, ref, act):
    ok, _, ratio = og.check(got, ref["c64"], ref["tau"], act)
    assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("kernel", [0, 1, 2])
@pytest.mark.parametrize("M", [1, 16, 64, 1024])
def test_mxint4_square(M, kernel, act):
    _check(*_run(M, 4096, 4096, act, None if kernel == 0 else dict(kernel=kernel)), act)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (5, 256, 1152), (37, 384, 640), (200, 256, 384)])
def test_mxint4_ragged(M, N, K, act):
    _check(*_run(M, N, K, act), act)
    _check(*_run(M, N, K, act, dict(kernel=1, tile_m=16 * (1 if M <= 16 else 2), tile_n=32)), act)
    _check(*_run(M, N, K, act, dict(kernel=2, tile_m=64, tile_n=128)), act)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("tuning", [dict(kernel=2, tile_m=64, tile_n=128, stages=2),
                                    dict(kernel=2, tile_m=128, tile_n=256, stages=4),
                                    dict(kernel=2, tile_m=64, tile_n=128, split_k=3),
                                    dict(kernel=1, split_k=4), dict(kernel=1, tile_m=16, tile_n=64, waves=4)])
def test_mxint4_tunings(tuning, act):
    _check(*_run(96, 512, 1536, act, tuning), act)


@pytest.mark.parametrize("kernel", [1, 2])
def test_mxint4_extreme_and_nan_scales(kernel):
    """Scales from 2^-127 (fp32 subnormal products) to 2^20, and one NaN code:
    its column is NaN in every row, every other output within tolerance."""
    M, N, K = 40, 256, 512
    d = datagen.w4a16_mxint4(M, N, K, act="bf16")
    e8 = d["e8m0"].copy()
    e8[:, 0] = 0                 # 2^-127
    e8[:, 1] = 147               # 2^20
    e8[7, 3] = 255               # NaN block in column 7
    d["e8m0"] = e8
    got, ref = _run(M, N, K, "bf16", dict(kernel=kernel), d=d)
    assert np.isnan(got[:, 7]).all() and np.isnan(ref["c64"][:, 7]).all()
    keep = np.ones(N, bool)
    keep[7] = False
    ok, _, ratio = og.check(got[:, keep], ref["c64"][:, keep], ref["tau"][:, keep], "bf16")
    assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"


def test_mxint4_gpu_repack_equals_host():
    _log("w4a16-mxint4 repack")
    d = datagen.w4a16_mxint4(1, 256, 1024)
    plan = hq.Plan(256, 1024, hq.w4a16_mxint4("bf16"), max_m=16)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    wh, mh = plan.repack_host(torch.from_numpy(d["codes"]), e8m0=torch.from_numpy(d["e8m0"]))
    torch.cuda.synchronize()
    assert torch.equal(w.cpu(), wh) and torch.equal(meta.cpu(), mh)
