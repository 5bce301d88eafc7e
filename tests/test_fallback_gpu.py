"""The fallback to 16-bit activations and Plan.linear on the GPU, against the
oracle.

* A description whose activation type the library does not run for those
  weights (NVFP4 or MXINT4 weights with fp8 activations, INT4 weights with
  per-group zero points and int8 activations) becomes a plan with 16-bit
  activations for the same weights (the pages' fallback to a higher-precision
  compute type); Plan.linear on 16-bit activations must match the oracle's
  16-bit-activation GEMM of the same weights.
* Plan.linear on a plan that does run 8-bit or MXFP4 activations quantises
  them with the library's quantiser kernels first: the activation codes must
  equal the oracle quantiser's bit for bit, and the product the oracle's GEMM
  of those codes.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_repack_amd as hq
import datagen
from oracle import gemm as og
from oracle import quant as oq
from oracle.formats import e4m3_value

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

NVFP4_FP8 = hq.QuantDesc(hq.FP4_E2M1, 4, 16, hq.FP8_E4M3, hq.ZP_NONE, 0, hq.FP8_E4M3, hq.ASCALE_PER_TOKEN_F32, hq.BF16)
MXINT4_FP8 = hq.QuantDesc(hq.I4, 4, 32, hq.E8M0, hq.ZP_NONE, 0, hq.FP8_E4M3, hq.ASCALE_PER_TOKEN_F32, hq.BF16)
INT4U4_I8 = hq.QuantDesc(hq.U4, 4, 128, hq.F16, hq.ZP_PER_GROUP_U4, 0, hq.INT8, hq.ASCALE_PER_TOKEN_F32, hq.F16)


def _log(msg):
    print(f"[gpu case] {msg}", flush=True)


def _assert_ok(got, ref, fmt, what):
    ok, _, ratio = og.check(got, ref["c64"], ref["tau"], fmt)
    assert ok.all(), f"{what}: {int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"


@pytest.mark.parametrize("M", [1, 16, 300])
def test_nvfp4_with_fp8_request_runs_bf16_activations(M):
    N, K = 512, 1024
    _log(f"fallback nvfp4 x fp8 -> bf16 M={M}")
    plan = hq.Plan(N, K, NVFP4_FP8, max_m=M)
    assert plan.fallback and plan.quant.act == hq.BF16
    d = datagen.w4a16_nvfp4(M, N, K, act="bf16")
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), torch.from_numpy(d["tscale"]).to(DEV),
                          e8m0=torch.from_numpy(d["e4m3"]).to(DEV))
    out = plan.linear(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    ref = og.gemm_nvfp4_w16(d["a"].double().numpy(), d["codes"], d["e4m3"], float(d["tscale"][0]), out_fmt="bf16")
    _assert_ok(out.double().cpu().numpy(), ref, "bf16", "nvfp4 fallback")


@pytest.mark.parametrize("M", [4, 64])
def test_mxint4_with_fp8_request_runs_bf16_activations(M):
    N, K = 256, 2048
    _log(f"fallback mxint4 x fp8 -> bf16 M={M}")
    plan = hq.Plan(N, K, MXINT4_FP8, max_m=M)
    assert plan.fallback and plan.quant.act == hq.BF16
    d = datagen.w4a16_mxint4(M, N, K, act="bf16")
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    out = plan.linear(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    ref = og.gemm_mxint4_w16(d["a"].double().numpy(), d["codes"], d["e8m0"], out_fmt="bf16")
    _assert_ok(out.double().cpu().numpy(), ref, "bf16", "mxint4 fallback")


@pytest.mark.parametrize("M", [2, 33, 256])
def test_int4_zero_points_with_int8_request_runs_f16_activations(M):
    N, K = 384, 1280
    _log(f"fallback int4-u4 x int8 -> f16 M={M}")
    plan = hq.Plan(N, K, INT4U4_I8, max_m=M)
    assert plan.fallback and plan.quant.act == hq.F16 and plan.quant.zp == hq.ZP_PER_GROUP_U4
    d = datagen.dense_w4a16(M, N, K, act="f16", zp="u4", key=(41,))
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV),
                          torch.from_numpy(d["zeros"]).to(DEV))
    out = plan.linear(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    ref = og.gemm_w4a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), d["zeros"], out_fmt="f16")
    _assert_ok(out.double().cpu().numpy(), ref, "f16", "int4 u4 fallback")


@pytest.mark.parametrize("kind", ["int8", "fp8", "mxfp4xfp8"])
@pytest.mark.parametrize("M", [1, 40, 512])
def test_linear_quantises_8_bit_activations(kind, M):
    N, K = 512, 2048
    _log(f"linear {kind} M={M}")
    rng = np.random.default_rng(M * 13 + len(kind))
    x = torch.from_numpy(rng.standard_normal((M, K))).to(torch.bfloat16)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes = datagen.pack_u4(q)
    if kind == "mxfp4xfp8":
        plan = hq.Plan(N, K, hq.w4a8_mxfp4(), max_m=M)
        e8 = (127 + rng.integers(-8, -3, size=(N, K // 32))).astype(np.uint8)
        w, meta = plan.repack(torch.from_numpy(codes).to(DEV), e8m0=torch.from_numpy(e8).to(DEV))
    else:
        plan = hq.Plan(N, K, hq.w4a8_int() if kind == "int8" else hq.w4a8_fp8(), max_m=M)
        scales = torch.from_numpy(rng.uniform(0.005, 0.02, size=(N, K // 128))).to(torch.float16)
        w, meta = plan.repack(torch.from_numpy(codes).to(DEV), scales.to(DEV))
    assert plan.fallback is None
    out = plan.linear(x.to(DEV), w, meta)
    torch.cuda.synchronize()
    # the activation codes the library produced: the oracle quantiser's, bit for bit
    qkind = "int8" if kind == "int8" else "fp8"
    ac, asc = oq.quantize_rows(x.float().numpy(), qkind)
    gc, gs = plan._act_buf[(torch.device(DEV), M)]
    assert np.array_equal(gc.cpu().numpy().view(ac.dtype), ac) and np.array_equal(gs.cpu().numpy(), asc)
    if kind == "int8":
        ref = og.gemm_int4_int8(ac, asc, codes, scales.double().numpy())
    elif kind == "fp8":
        ref = og.gemm_w4a16(e4m3_value(ac) * asc[:, None].astype(np.float64), codes, scales.double().numpy(), 8,
                            out_fmt="bf16")
    else:
        ref = og.gemm_mxfp4_fp8(ac, asc, codes, e8)
    _assert_ok(out.double().cpu().numpy(), ref, "bf16", f"linear {kind}")


@pytest.mark.parametrize("M", [3, 128])
def test_linear_quantises_mxfp4_activations(M):
    N, K = 256, 1024
    _log(f"linear w4a4 M={M}")
    rng = np.random.default_rng(M + 5)
    x = torch.from_numpy(rng.standard_normal((M, K)) * 2).to(torch.float16)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes = datagen.pack_u4(q)
    e8 = (127 + rng.integers(-8, -3, size=(N, K // 32))).astype(np.uint8)
    plan = hq.Plan(N, K, hq.w4a4_mxfp4(), max_m=M)
    w, meta = plan.repack(torch.from_numpy(codes).to(DEV), e8m0=torch.from_numpy(e8).to(DEV))
    out = plan.linear(x.to(DEV), w, meta)
    torch.cuda.synchronize()
    ac, ae = oq.mx_quantize_rows(x.double().numpy())
    ref = og.gemm_mxfp4_mxfp4(datagen.pack_u4(ac), ae, codes, e8)
    _assert_ok(out.double().cpu().numpy(), ref, "bf16", "linear w4a4")
