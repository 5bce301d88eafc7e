"""hq_gemm_noalloc on the GPU: the same result as hq_gemm, bit for bit, and the
oracle's within tolerance; calls in a row on the library's scratch (the second
smaller than the first); requests above the scratch rejected before any launch.
"""
import ctypes

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


class Case:
    def __init__(self, M, N, K, max_m=None, tuning=None):
        self.M, self.N, self.K = M, N, K
        self.d = datagen.dense_w4a16(M, N, K, act="bf16", zp="u4", key=(61,))
        self.plan = hq.Plan(N, K, hq.w4a16(act="bf16", zp="u4"), max_m=max_m or M, tuning=tuning)
        self.w, self.meta = self.plan.repack(torch.from_numpy(self.d["codes"]).to(DEV), self.d["scales"].to(DEV),
                                             torch.from_numpy(self.d["zeros"]).to(DEV))
        self.a = self.d["a"].to(DEV)

    def noalloc(self, m):
        out = torch.empty((m, self.N), dtype=torch.bfloat16, device=DEV)
        st = hq.lib().hq_gemm_noalloc(self.plan._h, m, self.a.data_ptr(), None, self.w.data_ptr(),
                                      self.meta.data_ptr(), out.data_ptr(), hq._stream_ptr(torch.device(DEV)))
        return st, out

    def with_workspace(self, m):
        return self.plan.gemm(self.a[:m].contiguous(), self.w, self.meta)

    def check(self, m, out):
        ref = og.gemm_w4a16(self.d["a"][:m].double().numpy(), self.d["codes"], self.d["scales"].double().numpy(),
                            self.d["zeros"], out_fmt="bf16")
        ok, _, ratio = og.check(out.double().cpu().numpy(), ref["c64"], ref["tau"], "bf16")
        assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance, max err/tau {ratio.max():.3g}"


def _same(case, m):
    _log(f"noalloc M={m} N={case.N} K={case.K} plan: {case.plan.describe(m)}")
    st, got = case.noalloc(m)
    assert st == hq.HQ_OK, hq.lib().hq_last_error().decode()
    want = case.with_workspace(m)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "hq_gemm_noalloc differs from hq_gemm"
    case.check(m, got)


def test_noalloc_matches_hq_gemm_on_calls_in_a_row():
    big = Case(64, 14336, 4096)                 # tiled kernel, K split 2: 7.3 MB of partials
    assert big.plan.workspace_bytes(64) > 0
    _same(big, 64)
    small = Case(16, 4096, 14336)               # skinny kernel, K split 4: 1 MB, a smaller input
    assert 0 < small.plan.workspace_bytes(16) < big.plan.workspace_bytes(64)
    _same(small, 16)
    _same(big, 37)                              # the first plan again with fewer rows
    _same(Case(1, 4096, 4096), 1)               # no K split: no scratch at all


def test_noalloc_rejects_partials_above_its_scratch():
    c = Case(256, 8192, 8192, tuning=dict(kernel=2, tile_m=128, tile_n=128, split_k=8))
    assert c.plan.workspace_bytes(256) > 16 << 20
    out = torch.zeros((256, 8192), dtype=torch.bfloat16, device=DEV)
    st = hq.lib().hq_gemm_noalloc(c.plan._h, 256, c.a.data_ptr(), None, c.w.data_ptr(), c.meta.data_ptr(),
                                  out.data_ptr(), hq._stream_ptr(torch.device(DEV)))
    torch.cuda.synchronize()
    assert st == hq.HQ_ERR_WORKSPACE and "library scratch" in hq.lib().hq_last_error().decode()
    assert int(out.view(torch.int16).abs().sum().item()) == 0  # nothing was launched
