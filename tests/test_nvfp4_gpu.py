"""W4A16-NVFP4 (NVFP4 weights, fp16 / bf16 activations) on the GPU against
the oracle.

Every output must lie within the oracle's tolerance (tau + half an output ulp,
oracle/gemm.py) on both kernels and the automatic choice, over decode and
prefill-sized M at N = K = 4096 (sampled rows for the large M), ragged shapes
spanning several tiles and the tile tunings; subnormal, negative and NaN
E4M3 block scales; the GPU repack equals the host repack byte for byte.
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
    _log(f"w4a16-nvfp4 M={M} N={N} K={K} act={act} tuning={tuning}")
    d = d or datagen.w4a16_nvfp4(M, N, K, act=act)
    plan = hq.Plan(N, K, hq.w4a16_nvfp4(act), max_m=M, tuning=tuning)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), torch.from_numpy(d["tscale"]).to(DEV),
                          e8m0=torch.from_numpy(d["e4m3"]).to(DEV))
    out = plan.gemm(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, min(M, 12)).astype(int))
    ref = og.gemm_nvfp4_w16(d["a"].double().numpy()[rows], d["codes"], d["e4m3"], float(d["tscale"][0]),
                            out_fmt=act)
    return out.double().cpu().numpy()[rows], ref


def _check(got, ref, act):
    ok, _, ratio = og.check(got, ref["c64"], ref["tau"], act)
    assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("kernel", [0, 1, 2])
@pytest.mark.parametrize("M", [1, 16, 64, 1024])
def test_nvfp4_square(M, kernel, act):
    _check(*_run(M, 4096, 4096, act, None if kernel == 0 else dict(kernel=kernel)), act)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (5, 256, 1152), (37, 384, 640), (200, 256, 384)])
def test_nvfp4_ragged(M, N, K, act):
    _check(*_run(M, N, K, act), act)
    _check(*_run(M, N, K, act, dict(kernel=1, tile_m=16 * (1 if M <= 16 else 2), tile_n=32)), act)
    _check(*_run(M, N, K, act, dict(kernel=2, tile_m=64, tile_n=128)), act)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("tuning", [dict(kernel=2, tile_m=64, tile_n=128, stages=2),
                                    dict(kernel=2, tile_m=128, tile_n=256, stages=4),
                                    dict(kernel=2, tile_m=64, tile_n=128, split_k=3),
                                    dict(kernel=1, split_k=4), dict(kernel=1, tile_m=16, tile_n=64, waves=4)])
def test_nvfp4_tunings(tuning, act):
    _check(*_run(96, 512, 1536, act, tuning), act)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("kernel", [1, 2])
def test_nvfp4_edge_scales(kernel, act):
    """Subnormal, negative and extreme E4M3 block scales, one NaN block
    scale: its column is NaN in every row, every other output in tolerance."""
    M, N, K = 40, 256, 512
    d = datagen.w4a16_nvfp4(M, N, K, act=act)
    e4 = d["e4m3"].copy()
    e4[:, 0] = 0x01          # 2^-9, the smallest subnormal
    e4[:, 1] = 0x07          # 7 * 2^-9
    e4[:, 2] = 0x7E          # 448, the largest normal
    e4[:, 3] = 0xB8          # -1
    e4[9, 5] = 0x7F          # NaN block in column 9
    d["e4m3"] = e4
    got, ref = _run(M, N, K, act, dict(kernel=kernel), d=d)
    assert np.isnan(got[:, 9]).all() and np.isnan(ref["c64"][:, 9]).all()
    keep = np.ones(N, bool)
    keep[9] = False
    ok, _, ratio = og.check(got[:, keep], ref["c64"][:, keep], ref["tau"][:, keep], act)
    assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"


def test_nvfp4_gpu_repack_equals_host():
    _log("w4a16-nvfp4 repack")
    d = datagen.w4a16_nvfp4(1, 256, 1024)
    plan = hq.Plan(256, 1024, hq.w4a16_nvfp4("bf16"), max_m=16)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), torch.from_numpy(d["tscale"]).to(DEV),
                          e8m0=torch.from_numpy(d["e4m3"]).to(DEV))
    wh, mh = plan.repack_host(torch.from_numpy(d["codes"]), torch.from_numpy(d["tscale"]),
                              e8m0=torch.from_numpy(d["e4m3"]))
    torch.cuda.synchronize()
    assert torch.equal(w.cpu(), wh) and torch.equal(meta.cpu(), mh)
