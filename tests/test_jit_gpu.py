"""Run-time specialised kernels (hq_plan_set_jit) on the GPU: every output
against the oracle and beside the precompiled kernel's output, for the skinny
and the tiled kernel over the formats and shapes of the decode, prefill and
W4A8 configurations (ragged shapes included), the exact int32 accumulators
of INT4 x int8 bit for bit, and the code-object cache (compile, memory hit,
disk hit) through the launch counters."""
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


def _pair(N, K, quant, M, cache, **kw):
    aot = hq.Plan(N, K, quant, max_m=M, **kw)
    jit = hq.Plan(N, K, quant, max_m=M, **kw)
    jit.set_jit(True, str(cache))
    assert aot.describe(M) == jit.describe(M)
    return aot, jit


def _check(out_jit, out_aot, ref, what):
    got = out_jit.double().cpu().numpy()
    ok, _, ratio = og.check(got, ref["c64"], ref["tau"], "bf16" if out_jit.dtype == torch.bfloat16 else "f16")
    assert ok.all(), f"{what}: {int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"
    same = float((out_jit == out_aot).float().mean())
    _log(f"{what}: max err/tau {ratio.max():.3g}, equal to the precompiled kernel's output: {same:.4f}")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (16, 4096, 4096), (64, 4096, 4096), (5, 14336, 4096),
                                   (64, 14336, 4096), (37, 384, 1280)])
def test_jit_w4a16_bf16_zero_points(M, N, K, tmp_path):
    _log(f"jit w4a16 bf16 u4 M={M} N={N} K={K}")
    d = datagen.dense_w4a16(M, N, K, act="bf16", zp="u4", key=(2,))
    aot, jit = _pair(N, K, hq.w4a16(act="bf16", zp="u4"), M, tmp_path)
    w, meta = aot.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV), torch.from_numpy(d["zeros"]).to(DEV))
    a = d["a"].to(DEV)
    s0 = hq.jit_stats()
    oa = aot.gemm(a, w, meta)
    oj = jit.gemm(a, w, meta)
    torch.cuda.synchronize()
    assert hq.jit_stats()["launches"] == s0["launches"] + 1
    ref = og.gemm_w4a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), d["zeros"], out_fmt="bf16")
    _check(oj, oa, ref, f"w4a16 bf16 M={M} N={N} K={K} ({jit.describe(M)})")


@pytest.mark.parametrize("M,N,K", [(1024, 4096, 4096), (300, 512, 1024)])
def test_jit_w4a16_f16_prefill(M, N, K, tmp_path):
    _log(f"jit w4a16 f16 M={M} N={N} K={K}")
    d = datagen.dense_w4a16(M, N, K, act="f16", zp="fixed", key=(3,))
    aot, jit = _pair(N, K, hq.w4a16("f16"), M, tmp_path)
    w, meta = aot.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
    oa = aot.gemm(d["a"].to(DEV), w, meta)
    oj = jit.gemm(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    ref = og.gemm_w4a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), 8, out_fmt="f16")
    _check(oj, oa, ref, f"w4a16 f16 M={M} ({jit.describe(M)})")


@pytest.mark.parametrize("M", [16, 1024])
def test_jit_w4a8_mxfp4(M, tmp_path):
    N, K = 4096, 7168
    _log(f"jit w4a8 mxfp4 M={M}")
    d = datagen.w4a8_mxfp4(M, N, K)
    aot, jit = _pair(N, K, hq.w4a8_mxfp4(), M, tmp_path)
    w, meta = aot.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    a, s = d["a_codes"].to(DEV), d["a_scale"].to(DEV)
    oa = aot.gemm(a, w, meta, a_scale=s)
    oj = jit.gemm(a, w, meta, a_scale=s)
    torch.cuda.synchronize()
    ref = og.gemm_mxfp4_fp8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["e8m0"])
    _check(oj, oa, ref, f"mxfp4 M={M} ({jit.describe(M)})")


@pytest.mark.parametrize("M,N,K", [(7, 512, 2048), (200, 384, 1152)])
def test_jit_int4_int8_accumulators_exact(M, N, K, tmp_path):
    _log(f"jit w4a8 int i32 M={M} N={N} K={K}")
    d = datagen.w4a8_int(M, N, K)
    jit = hq.Plan(N, K, hq.w4a8_int(), max_m=M, epi="i32_acc")
    jit.set_jit(True, str(tmp_path))
    w, meta = jit.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
    P = jit.gemm(d["a_codes"].to(DEV), w, meta, a_scale=d["a_scale"].to(DEV))
    torch.cuda.synchronize()
    ref = og.gemm_int4_int8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["scales"].double().numpy())
    assert np.array_equal(P.cpu().numpy().astype(np.int64), ref["P"])
    f = hq.Plan(N, K, hq.w4a8_int(), max_m=M)
    f.set_jit(True, str(tmp_path))
    out = f.gemm(d["a_codes"].to(DEV), w, meta, a_scale=d["a_scale"].to(DEV))
    torch.cuda.synchronize()
    ok, _, ratio = og.check(out.double().cpu().numpy(), ref["c64"], ref["tau"], "bf16")
    assert ok.all(), f"max err/tau {ratio.max():.3g}"


def test_jit_cache_compile_memory_and_disk(tmp_path):
    N, K, M = 2048, 2048, 9
    d = datagen.dense_w4a16(M, N, K, act="bf16", zp="u4", key=(19,))
    a = d["a"].to(DEV)
    p = hq.Plan(N, K, hq.w4a16(act="bf16", zp="u4"), max_m=M)
    w, meta = p.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV), torch.from_numpy(d["zeros"]).to(DEV))
    ref = og.gemm_w4a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), d["zeros"], out_fmt="bf16")
    p.set_jit(True, str(tmp_path / "first"))
    s0 = hq.jit_stats()
    o1 = p.gemm(a, w, meta)                            # compiled now
    s1 = hq.jit_stats()
    assert s1["compiles"] == s0["compiles"] + 1 and (tmp_path / "first" / (p.jit_cache_key(M) + ".co")).exists()
    o2 = p.gemm(a, w, meta)                            # already loaded
    s2 = hq.jit_stats()
    assert s2["memory_hits"] == s1["memory_hits"] + 1 and s2["compiles"] == s1["compiles"]
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for o in (o1, o2):
        ok, _, ratio = og.check(o.double().cpu().numpy(), ref["c64"], ref["tau"], "bf16")
        assert ok.all()
    # a shape not run in this process yet, prepared ahead without a device: loaded from disk
    q = hq.Plan(N, K, hq.w4a16(act="bf16", zp="u4"), max_m=M)
    q.set_jit(True, str(tmp_path / "ahead"))
    q.set_tuning(M, dict(kernel=1, tile_m=16, tile_n=32, waves=4, split_k=1, stages=4))
    q.jit_prepare(M)
    s3 = hq.jit_stats()
    o3 = q.gemm(a, w, meta)
    s4 = hq.jit_stats()
    assert s4["disk_hits"] == s3["disk_hits"] + 1 and s4["compiles"] == s3["compiles"]
    torch.cuda.synchronize()
    ok, _, ratio = og.check(o3.double().cpu().numpy(), ref["c64"], ref["tau"], "bf16")
    assert ok.all()
    q.set_jit(False)                                   # back to the precompiled kernel
    s5 = hq.jit_stats()
    q.gemm(a, w, meta)
    assert hq.jit_stats()["launches"] == s5["launches"]
