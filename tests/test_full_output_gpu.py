"""Every output of the large configurations the float64 oracle still computes in
seconds, on the GPU against the oracle (the other GPU tests sample rows of
these sizes):

* dense W4A16 prefill, M = 1024, N = K = 8192, fp16, zero point 8: all 8.4 M
  outputs;
* W4A8 at M = 1024, N = 4096, K = 7168: MXFP4 x fp8 and INT4 x int8, all 4.2 M
  outputs each.  For INT4 x int8 the oracle's value is the definition
  C = s_a * sum_g s[n,g] * P[m,n,g] evaluated as one float64 product of the
  int8 codes and the exactly dequantised weights (every P is an integer below
  2^17, so the float64 sum is exact to its last bit); the integer P itself is
  compared bit for bit with the oracle's int64 accumulators at the other sizes
  (tests/test_gemm_gpu.py).

The 256-expert MoE layer at T = 512 on all tokens is in tests/test_moe_gpu.py.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_repack_amd as hq
import datagen
from oracle import gemm as og
from oracle.formats import int8_value

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _log(msg):
    print(f"[gpu case] {msg}", flush=True)


def _assert_all(got, ref, fmt, what):
    ok, lit, ratio = og.check(got, ref["c64"], ref["tau"], fmt)
    _log(f"{what}: {ok.size} outputs, max err/tau {ratio.max():.3g}, literal-tau pass {lit.mean():.5f}")
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} outputs outside tolerance, max err/tau {ratio.max():.3g}"


def test_prefill_fp16_m1024_every_output():
    M, N, K = 1024, 8192, 8192
    _log(f"full-output prefill M={M} N={N} K={K}")
    d = datagen.dense_w4a16(M, N, K, act="f16", zp="fixed", key=(3,))
    plan = hq.Plan(N, K, hq.w4a16("f16"), max_m=M)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
    out = plan.gemm(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    ref = og.gemm_w4a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), 8, out_fmt="f16")
    _assert_all(out.double().cpu().numpy(), ref, "f16", f"prefill ({plan.describe(M)})")


def test_w4a8_mxfp4_fp8_m1024_every_output():
    M, N, K = 1024, 4096, 7168
    _log(f"full-output w4a8 mxfp4 x fp8 M={M}")
    d = datagen.w4a8_mxfp4(M, N, K)
    plan = hq.Plan(N, K, hq.w4a8_mxfp4(), max_m=M)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    out = plan.gemm(d["a_codes"].to(DEV), w, meta, a_scale=d["a_scale"].to(DEV))
    torch.cuda.synchronize()
    ref = og.gemm_mxfp4_fp8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["e8m0"])
    _assert_all(out.double().cpu().numpy(), ref, "bf16", f"w4a8 mxfp4 ({plan.describe(M)})")


def test_w4a8_int4_int8_m1024_every_output():
    M, N, K = 1024, 4096, 7168
    _log(f"full-output w4a8 int4 x int8 M={M}")
    d = datagen.w4a8_int(M, N, K)
    plan = hq.Plan(N, K, hq.w4a8_int(), max_m=M)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
    out = plan.gemm(d["a_codes"].to(DEV), w, meta, a_scale=d["a_scale"].to(DEV))
    torch.cuda.synchronize()
    a_val = int8_value(d["a_codes"].numpy()) * d["a_scale"].numpy().astype(np.float64)[:, None]
    ref = og.gemm_w4a16(a_val, d["codes"], d["scales"].double().numpy(), 8, out_fmt="bf16")
    _assert_all(out.double().cpu().numpy(), ref, "bf16", f"w4a8 int ({plan.describe(M)})")
