"""W3A16 (INT3 weights, fp16 / bf16 activations) on the GPU against the oracle.

Every output must lie within the oracle's tolerance (tau + half an output ulp,
oracle/gemm.py) on both kernels and the automatic choice, over decode and
prefill-sized M at N = K = 4096 (sampled rows for the large M), ragged shapes
spanning several tiles, every fixed zero point and the tile tunings; the GPU
repack must equal the host repack byte for byte.
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


def _run(M, N, K, act, tuning=None, zp=4):
    _log(f"w3a16 M={M} N={N} K={K} act={act} zp={zp} tuning={tuning}")
    d = datagen.dense_w3a16(M, N, K, act=act)
    plan = hq.Plan(N, K, hq.w3a16(act, zp_value=zp), max_m=M, tuning=tuning)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
    out = plan.gemm(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, min(M, 12)).astype(int))
    ref = og.gemm_w3a16(d["a"].double().numpy()[rows], d["codes"], d["scales"].double().numpy(), zp, out_fmt=act)
    ok, _, ratio = og.check(out.double().cpu().numpy()[rows], ref["c64"], ref["tau"], act)
    assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("kernel", [0, 1, 2])
@pytest.mark.parametrize("M", [1, 16, 64, 1024])
def test_w3a16_square(M, kernel, act):
    _run(M, 4096, 4096, act, None if kernel == 0 else dict(kernel=kernel))


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (5, 256, 1152), (37, 384, 640), (200, 256, 384)])
def test_w3a16_ragged(M, N, K, act):
    _run(M, N, K, act)
    _run(M, N, K, act, dict(kernel=1, tile_m=16 * (1 if M <= 16 else 2), tile_n=32), zp=0)
    _run(M, N, K, act, dict(kernel=2, tile_m=64, tile_n=128), zp=7)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("tuning", [dict(kernel=2, tile_m=64, tile_n=128, stages=2),
                                    dict(kernel=2, tile_m=128, tile_n=256, stages=4),
                                    dict(kernel=2, tile_m=64, tile_n=128, split_k=3),
                                    dict(kernel=1, split_k=4), dict(kernel=1, tile_m=16, tile_n=64, waves=4)])
def test_w3a16_tunings(tuning, act):
    _run(96, 512, 1536, act, tuning, zp=5)


def test_w3a16_gpu_repack_equals_host():
    _log("w3a16 repack")
    d = datagen.dense_w3a16(1, 256, 1024)
    plan = hq.Plan(256, 1024, hq.w3a16("bf16"), max_m=16)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
    wh, mh = plan.repack_host(torch.from_numpy(d["codes"]), d["scales"])
    torch.cuda.synchronize()
    assert torch.equal(w.cpu(), wh) and torch.equal(meta.cpu(), mh)
