"""Autotuning on the GPU: hq_plan_autotune times the candidate execution
choices, installs the fastest for that m, and the plan's later calls use it.

Each case checks that the installed choice is the timed minimum (never slower
than the choice in force before, which is one of the timed candidates), that
the plan reports it for that m only, and that the GEMM run with it stays
within the oracle's tolerance (tau + half an output ulp, oracle/gemm.py).
The tuning cache round-trips through its JSON file into a fresh plan.
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


def _check_result(plan, m, r):
    assert r["candidates"] >= 4
    assert r["best_us"] <= r["current_us"]
    assert r["best_us"] > 0
    assert plan.get_tuning(m) == (r["tuning"], True)
    other = m + 1 if m < plan.max_m else m - 1
    assert not plan.get_tuning(other)[1]


@pytest.mark.parametrize("M,N,K,act", [(1, 4096, 4096, "bf16"), (16, 2048, 4096, "f16"), (200, 1024, 2048, "bf16")])
def test_autotune_w4a16(M, N, K, act):
    _log(f"autotune w4a16 M={M} N={N} K={K} act={act}")
    d = datagen.dense_w4a16(M, N, K, act=act, zp="u4")
    plan = hq.Plan(N, K, hq.w4a16(act, zp="u4"), max_m=max(M, 2))
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV),
                          torch.from_numpy(d["zeros"]).to(DEV))
    a = d["a"].to(DEV)
    r = plan.autotune(a, w, meta, reps=4, flush_bytes=256 << 20)
    _log(f"  {r}")
    _check_result(plan, M, r)
    assert plan.describe(M).startswith("kernel=" + ("skinny" if r["tuning"]["kernel"] == 1 else "tiled"))
    out = plan.gemm(a, w, meta)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, min(M, 12)).astype(int))
    ref = og.gemm_w4a16(d["a"].double().numpy()[rows], d["codes"], d["scales"].double().numpy(), d["zeros"],
                        out_fmt=act)
    ok, _, ratio = og.check(out.double().cpu().numpy()[rows], ref["c64"], ref["tau"], act)
    assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"


def test_autotune_w4a8_mxfp4():
    M, N, K = 16, 1024, 7168
    _log(f"autotune w4a8-mxfp4 M={M} N={N} K={K}")
    d = datagen.w4a8_mxfp4(M, N, K)
    plan = hq.Plan(N, K, hq.w4a8_mxfp4(), max_m=64)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    a, sa = d["a_codes"].to(DEV), d["a_scale"].to(DEV)
    r = plan.autotune(a, w, meta, a_scale=sa, reps=4, flush_bytes=0)
    _log(f"  {r}")
    _check_result(plan, M, r)
    out = plan.gemm(a, w, meta, a_scale=sa)
    torch.cuda.synchronize()
    ref = og.gemm_mxfp4_fp8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["e8m0"])
    ok, _, ratio = og.check(out.double().cpu().numpy(), ref["c64"], ref["tau"], "bf16")
    assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"


def test_tuning_cache_round_trip(tmp_path):
    M, N, K = 4, 1024, 1024
    _log(f"tuning cache M={M} N={N} K={K}")
    d = datagen.dense_w4a16(M, N, K, act="bf16")
    path = str(tmp_path / "tunings.json")
    plan = hq.Plan(N, K, hq.w4a16("bf16"), max_m=64)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
    a = d["a"].to(DEV)
    cache = hq.TuningCache(path)
    r1 = cache.tune(plan, a, w, meta, reps=3, flush_bytes=0)
    assert not r1["cached"]
    fresh = hq.Plan(N, K, hq.w4a16("bf16"), max_m=64)
    assert hq.TuningCache(path).apply(fresh, DEV) == 1
    assert fresh.get_tuning(M) == (r1["tuning"], True)
    r2 = hq.TuningCache(path).tune(fresh, a, w, meta)
    assert r2["cached"] and r2["tuning"] == r1["tuning"]
    other = hq.Plan(N, K, hq.w4a16("f16"), max_m=64)   # another format: no entry applies
    assert hq.TuningCache(path).apply(other, DEV) == 0
