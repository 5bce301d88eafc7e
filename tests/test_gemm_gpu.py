"""Dense GEMM parity on the GPU: the HIP path (through the C ABI) against the
CPU oracle, element by element, on the same seeded inputs.

Bar: every float output within tau + half an output ulp (the tolerance rule
in oracle/gemm.py), int32 accumulators bit-exact.  Shapes: the dense
workloads (M=16 N=256 K=512 fp16; the decode sweep M in {1,4,16,64} x
(N,K) in {(4096,4096),(14336,4096),(4096,14336)} bf16 with uint4 zero points;
W4A8 at N=4096 K=7168 for M in {1,16,128,1024}), ragged sizes, single-group
K, every tuning knob, and the degenerate m = 0.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_repack_amd as hq
import datagen
from oracle import gemm as og
from oracle.formats import e4m3_value, int8_value

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _log(msg):
    print(f"[gpu case] {msg}", flush=True)


def _assert_ok(out, ref, fmt, what):
    ok, literal, ratio = og.check(out, ref["c64"], ref["tau"], fmt)
    bad = int((~ok).sum())
    assert bad == 0, f"{what}: {bad}/{ok.size} outputs outside tolerance, max err/tau {ratio.max():.3g}"
    return ratio.max(), float(literal.mean())


# ----------------------------------------------------------------- W4A16 --

_ref_cache = {}


def w4a16_case(M, N, K, act, zp, key=(2,)):
    ck = (M, N, K, act, zp, key)
    if ck not in _ref_cache:
        d = datagen.dense_w4a16(M, N, K, act=act, zp=zp, key=key)
        zeros = d["zeros"] if zp == "u4" else 8
        ref = og.gemm_w4a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), zeros,
                            out_fmt=act)
        ref.pop("w")
        _ref_cache.clear()
        _ref_cache[ck] = (d, ref)
    return _ref_cache[ck]


def run_w4a16(M, N, K, act="bf16", zp="u4", tuning=None, key=(2,), max_m=None):
    _log(f"w4a16 M={M} N={N} K={K} act={act} zp={zp} tuning={tuning}")
    d, ref = w4a16_case(M, N, K, act, zp, key)
    plan = hq.Plan(N, K, hq.w4a16(act=act, zp=zp), max_m=max_m or max(M, 1), tuning=tuning)
    codes = torch.from_numpy(d["codes"]).to(DEV)
    zeros = torch.from_numpy(d["zeros"]).to(DEV) if zp == "u4" else None
    w, meta = plan.repack(codes, d["scales"].to(DEV), zeros)
    out = plan.gemm(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    return _assert_ok(out.double().cpu().numpy(), ref, act, f"w4a16 M={M} N={N} K={K}")


def test_dense_fp16_symmetric_small():
    # M=16, N=256, K=512, fp16 activations / scales / output, zero point 8
    run_w4a16(16, 256, 512, act="f16", zp="fixed", key=(1,))


@pytest.mark.parametrize("NK", [(4096, 4096), (14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_decode_sweep_bf16_uint4_zeros(M, NK):
    run_w4a16(M, NK[0], NK[1], act="bf16", zp="u4")


@pytest.mark.parametrize("M,N,K", [(5, 48, 384), (17, 96, 640), (33, 64, 1024), (63, 272, 512),
                                   (1, 16, 128), (7, 32, 128), (100, 256, 512), (130, 80, 256)])
@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_ragged_and_single_group(M, N, K, act):
    run_w4a16(M, N, K, act=act, zp="u4")


@pytest.mark.parametrize("tuning", [
    dict(split_k=1), dict(split_k=2), dict(split_k=4), dict(split_k=16), dict(split_k=64),
    dict(waves=1), dict(waves=2), dict(waves=8), dict(stages=4), dict(tile_n=16), dict(tile_n=64),
    dict(tile_n=32, split_k=8, waves=8, stages=4), dict(tile_m=32), dict(tile_m=64, tile_n=16),
])
def test_tuning_knobs(tuning):
    run_w4a16(16, 512, 2048, act="bf16", zp="u4", tuning=tuning)
    run_w4a16(16, 512, 2048, act="f16", zp="fixed", tuning=tuning)


@pytest.mark.parametrize("tuning", [
    None, dict(split_k=2), dict(split_k=3), dict(split_k=16), dict(waves=4), dict(waves=16), dict(stages=4),
    dict(tile_n=32), dict(tile_n=64), dict(tile_n=64, stages=4, split_k=2),
])
@pytest.mark.parametrize("M", [1, 3, 4])
def test_staged_activations(M, tuning):
    # up to 4 rows of 16-bit activations are copied into LDS once per
    # workgroup: split ranges whose byte span is not a whole KiB (K = 640, five
    # groups; uneven splits), every wave count, ring depth and column width
    run_w4a16(M, 256, 640, act="bf16", zp="u4", tuning=tuning)
    run_w4a16(M, 512, 2048, act="f16", zp="fixed", tuning=tuning)


def test_m_zero_is_noop_and_calls_repeat():
    N, K = 256, 1024
    d, ref = w4a16_case(16, N, K, "bf16", "u4")
    plan = hq.Plan(N, K, hq.w4a16(act="bf16", zp="u4"), max_m=16, tuning=dict(split_k=4))
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV),
                          torch.from_numpy(d["zeros"]).to(DEV))
    a = d["a"].to(DEV)
    empty = plan.gemm(a[:0], w, meta)
    assert empty.shape == (0, N)
    outs = [plan.gemm(a, w, meta) for _ in range(3)]  # every call rewrites its partials
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, outs[0])  # deterministic reduction order
    _assert_ok(outs[0].double().cpu().numpy(), ref, "bf16", "repeat")
    # a smaller m on the same workspace
    small = plan.gemm(a[:3], w, meta)
    torch.cuda.synchronize()
    assert torch.equal(small, outs[0][:3])


@pytest.mark.parametrize("quant", ["w4a16_u4", "w4a8_int", "w4a8_fp8", "mxfp4"])
def test_device_repack_matches_host_repack(quant):
    N, K = 96, 640
    rng = np.random.default_rng(11)
    codes = torch.from_numpy(datagen.pack_u4(rng.integers(0, 16, size=(N, K), dtype=np.uint8)))
    scales = torch.from_numpy(rng.uniform(0.005, 0.02, size=(N, K // 128))).to(torch.float16)
    zeros = torch.from_numpy(rng.integers(0, 16, size=(N, K // 128), dtype=np.uint8))
    e8 = torch.from_numpy(rng.integers(119, 124, size=(N, K // 32), dtype=np.uint8))
    q = {"w4a16_u4": hq.w4a16("f16", zp="u4"), "w4a8_int": hq.w4a8_int(), "w4a8_fp8": hq.w4a8_fp8(),
         "mxfp4": hq.w4a8_mxfp4()}[quant]
    plan = hq.Plan(N, K, q, max_m=1)
    kw = dict(e8m0=e8) if quant == "mxfp4" else dict(scales=scales, zeros=zeros if quant == "w4a16_u4" else None)
    wh, mh = plan.repack_host(codes, **kw)
    wd, md = plan.repack(codes.to(DEV), **{k: (v.to(DEV) if v is not None else None) for k, v in kw.items()})
    torch.cuda.synchronize()
    assert torch.equal(wd.cpu(), wh) and torch.equal(md.cpu(), mh)


# ------------------------------------------------------------------ W4A8 --

def _sample_rows(M, n=48, seed=0):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), n - 2, replace=False)]))


@pytest.mark.parametrize("M", [1, 16, 128, 1024])
def test_w4a8_int_accumulators_exact_and_output(M):
    N, K = 4096, 7168
    _log(f"w4a8-int M={M} N={N} K={K}")
    d = datagen.w4a8_int(M, N, K)
    a_codes, a_scale = d["a_codes"], d["a_scale"]
    rows = _sample_rows(M)
    codes = torch.from_numpy(d["codes"]).to(DEV)
    # float output
    plan = hq.Plan(N, K, hq.w4a8_int(), max_m=M)
    w, meta = plan.repack(codes, d["scales"].to(DEV))
    out = plan.gemm(a_codes.to(DEV), w, meta, a_scale=a_scale.to(DEV))
    # exact per-group int32 accumulators
    pacc = hq.Plan(N, K, hq.w4a8_int(), max_m=M, epi="i32_acc")
    P = pacc.gemm(a_codes.to(DEV), w, meta, a_scale=a_scale.to(DEV))
    torch.cuda.synchronize()
    ref = og.gemm_int4_int8(a_codes.numpy()[rows], a_scale.numpy()[rows], d["codes"],
                            d["scales"].double().numpy(), out_fmt="bf16")
    assert np.array_equal(P.cpu().numpy()[rows].astype(np.int64), ref["P"])
    _assert_ok(out.double().cpu().numpy()[rows], ref, "bf16", f"w4a8-int M={M}")


@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("M", [1, 16, 128, 1024])
def test_w4a8_mxfp4(M, kernel):
    N, K = 4096, 7168
    _log(f"w4a8-mxfp4 M={M} N={N} K={K} kernel={kernel}")
    d = datagen.w4a8_mxfp4(M, N, K)
    rows = _sample_rows(M)
    plan = hq.Plan(N, K, hq.w4a8_mxfp4(), max_m=M, tuning=dict(kernel=kernel))
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    out = plan.gemm(d["a_codes"].to(DEV), w, meta, a_scale=d["a_scale"].to(DEV))
    torch.cuda.synchronize()
    ref = og.gemm_mxfp4_fp8(d["a_codes"].numpy()[rows], d["a_scale"].numpy()[rows], d["codes"], d["e8m0"])
    _assert_ok(out.double().cpu().numpy()[rows], ref, "bf16", f"mxfp4 M={M}")


def _fp8_oracle(a_codes, a_scale, codes, scales, zeros):
    """INT4 x fp8: dequantised activations (code value * row scale) through the
    W4A16 oracle definition C = A . ((q - z) s)^T."""
    a = e4m3_value(a_codes) * np.asarray(a_scale, dtype=np.float64)[:, None]
    return og.gemm_w4a16(a, codes, scales, zeros, out_fmt="bf16")


@pytest.mark.parametrize("M,N,K,zp", [(1, 512, 7168, "fixed"), (16, 4096, 7168, "fixed"),
                                      (37, 256, 1024, "u4"), (128, 512, 256, "fixed")])
def test_w4a8_fp8_int4_weights(M, N, K, zp):
    _log(f"w4a8-fp8 M={M} N={N} K={K} zp={zp}")
    rng = np.random.default_rng(M * 7 + N)
    a32 = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    a_codes, a_scale = datagen.quant_per_token(a32, "fp8")
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes = datagen.pack_u4(q)
    scales = torch.from_numpy(rng.uniform(0.005, 0.02, size=(N, K // 128))).to(torch.float16)
    zeros = rng.integers(6, 10, size=(N, K // 128), dtype=np.uint8) if zp == "u4" else None
    plan = hq.Plan(N, K, hq.w4a8_fp8(zp=zp), max_m=M)
    w, meta = plan.repack(torch.from_numpy(codes).to(DEV), scales.to(DEV),
                          torch.from_numpy(zeros).to(DEV) if zeros is not None else None)
    out = plan.gemm(a_codes.to(DEV), w, meta, a_scale=a_scale.to(DEV))
    torch.cuda.synchronize()
    ref = _fp8_oracle(a_codes.numpy(), a_scale.numpy(), codes, scales.double().numpy(),
                      zeros if zeros is not None else 8)
    _assert_ok(out.double().cpu().numpy(), ref, "bf16", f"w4a8-fp8 M={M}")


def test_int8_activation_extremes():
    # rows of -128 / 127 codes against all-0 / all-15 weights: the int32 path at its range limits
    M, N, K = 4, 32, 256
    a = np.zeros((M, K), dtype=np.int8)
    a[0] = -128
    a[1] = 127
    a[2, ::2] = -128
    a[3] = np.arange(K) % 255 - 127
    q = np.zeros((N, K), dtype=np.uint8)
    q[16:] = 15
    q[8:16, ::3] = 15
    codes = datagen.pack_u4(q)
    scales = torch.ones(N, K // 128, dtype=torch.float16)
    plan = hq.Plan(N, K, hq.w4a8_int(), max_m=M, epi="i32_acc")
    w, meta = plan.repack(torch.from_numpy(codes).to(DEV), scales.to(DEV))
    P = plan.gemm(torch.from_numpy(a).to(DEV), w, meta, a_scale=torch.ones(M, device=DEV))
    torch.cuda.synchronize()
    ref = og.int_accumulators(a.view(np.uint8), codes)
    assert np.array_equal(P.cpu().numpy().astype(np.int64), ref)
    assert int8_value(np.array([128], np.uint8))[0] == -128


# --------------------------------------------------------- tiled kernel --

def _w4a16_sampled(M, N, K, act, zp, tuning=None, key=(3,)):
    _log(f"w4a16 sampled M={M} N={N} K={K} act={act} zp={zp} tuning={tuning}")
    d = datagen.dense_w4a16(M, N, K, act=act, zp=zp, key=key)
    rows = _sample_rows(M)
    zeros = d["zeros"] if zp == "u4" else 8
    plan = hq.Plan(N, K, hq.w4a16(act=act, zp=zp), max_m=M, tuning=tuning)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV),
                          torch.from_numpy(d["zeros"]).to(DEV) if zp == "u4" else None)
    out = plan.gemm(d["a"].to(DEV), w, meta)
    torch.cuda.synchronize()
    ref = og.gemm_w4a16(d["a"].double().numpy()[rows], d["codes"], d["scales"].double().numpy(), zeros,
                        out_fmt=act)
    return plan.describe(M), _assert_ok(out.double().cpu().numpy()[rows], ref, act, f"w4a16 M={M}")


@pytest.mark.parametrize("M", [1024, 4096])
def test_prefill_fp16_symmetric(M):
    # M in {1024, 4096}, N = K = 8192, fp16, zero point 8 (sampled rows)
    desc, _ = _w4a16_sampled(M, 8192, 8192, "f16", "fixed")
    assert "kernel=tiled" in desc


@pytest.mark.parametrize("tuning", [dict(kernel=2, tile_m=64, tile_n=128), dict(kernel=2, tile_m=64, tile_n=256),
                                    dict(kernel=2, tile_m=128, tile_n=128), dict(kernel=2, tile_m=128, tile_n=256)])
@pytest.mark.parametrize("act,zp", [("f16", "fixed"), ("bf16", "u4"), ("f16", "u4"), ("bf16", "fixed")])
def test_tiled_w4a16_shapes(tuning, act, zp):
    for (M, N, K) in [(200, 512, 1024), (1, 256, 128), (129, 768, 384)]:
        run_w4a16(M, N, K, act=act, zp=zp, tuning=tuning)


@pytest.mark.parametrize("stages", [2, 4, 5])
@pytest.mark.parametrize("tuning", [dict(kernel=2, tile_m=64, tile_n=128), dict(kernel=2, tile_m=128, tile_n=256),
                                    dict(kernel=2, tile_m=64, tile_n=256, split_k=3)])
@pytest.mark.parametrize("act,zp", [("f16", "fixed"), ("bf16", "u4")])
def test_tiled_deeper_pipeline(stages, tuning, act, zp):
    # 2-, 4- and 5-group load pipelines (G = 1, 3, 8, 11 groups: shorter
    # than, equal to and longer than the pipeline)
    for (M, N, K) in [(70, 512, 128), (130, 256, 384), (64, 512, 1024), (200, 256, 1408)]:
        run_w4a16(M, N, K, act=act, zp=zp, tuning=dict(tuning, stages=stages))


@pytest.mark.parametrize("split", [2, 3, 5, 8])
@pytest.mark.parametrize("act,zp", [("f16", "fixed"), ("bf16", "u4")])
def test_tiled_split_k(split, act, zp):
    # K split over workgroups + the second-pass reduce: an even split, uneven
    # ones (G = 16 or 10 groups), ragged M, both tile widths
    for (M, N, K, tn) in [(64, 512, 2048, 128), (40, 256, 1280, 256), (97, 384, 2048, 128)]:
        run_w4a16(M, N, K, act=act, zp=zp, tuning=dict(kernel=2, tile_m=64, tile_n=tn, split_k=split))


def test_tiled_split_k_w4a8_formats():
    M, N, K = 48, 256, 2048
    for tun in (dict(kernel=2, tile_m=64, tile_n=128, split_k=4), dict(kernel=2, tile_m=128, tile_n=256, split_k=3)):
        _log(f"tiled split w4a8 {tun}")
        d = datagen.w4a8_int(M, N, K)
        plan = hq.Plan(N, K, hq.w4a8_int(), max_m=M, tuning=tun)
        assert "split_k=" + str(tun["split_k"]) in plan.describe(M)
        w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
        out = plan.gemm(d["a_codes"].to(DEV), w, meta, a_scale=d["a_scale"].to(DEV))
        torch.cuda.synchronize()
        ref = og.gemm_int4_int8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["scales"].double().numpy())
        _assert_ok(out.double().cpu().numpy(), ref, "bf16", "split w4a8-int")
        d = datagen.w4a8_mxfp4(M, N, K)
        plan = hq.Plan(N, K, hq.w4a8_mxfp4(), max_m=M, tuning=tun)
        w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
        out = plan.gemm(d["a_codes"].to(DEV), w, meta, a_scale=d["a_scale"].to(DEV))
        torch.cuda.synchronize()
        ref = og.gemm_mxfp4_fp8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["e8m0"])
        _assert_ok(out.double().cpu().numpy(), ref, "bf16", "split w4a8-mxfp4")


@pytest.mark.parametrize("group", [1, 3, 8, 64])
def test_tiled_launch_order(group):
    # every tile computed once whatever the launch order: 5 x 6 tiles of 64 x 128
    # (a partial last row tile, a partial last group for 3 and 8, one group for 64)
    M, N, K = 300, 768, 1024
    _log(f"tiled launch order tile_group={group}")
    d = datagen.w4a8_mxfp4(M, N, K)
    plan = hq.Plan(N, K, hq.w4a8_mxfp4(), max_m=M, tuning=dict(kernel=2, tile_m=64, tile_n=128, tile_group=group))
    assert f"tile_group={group}" in plan.describe(M)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), e8m0=torch.from_numpy(d["e8m0"]).to(DEV))
    out = plan.gemm(d["a_codes"].to(DEV), w, meta, a_scale=d["a_scale"].to(DEV))
    torch.cuda.synchronize()
    ref = og.gemm_mxfp4_fp8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["e8m0"])
    _assert_ok(out.double().cpu().numpy(), ref, "bf16", f"launch order {group}")
    run_w4a16(M, N, K, act="f16", zp="fixed", tuning=dict(kernel=2, tile_m=128, tile_n=256, tile_group=group))


@pytest.mark.parametrize("tuning", [dict(kernel=2, tile_m=64, tile_n=256), dict(kernel=2, tile_m=128, tile_n=256),
                                    dict(kernel=2, tile_m=128, tile_n=128)])
def test_tiled_w4a8(tuning):
    M, N, K = 300, 512, 1024
    _log(f"tiled w4a8 {tuning}")
    # INT4 x INT8
    d = datagen.w4a8_int(M, N, K)
    plan = hq.Plan(N, K, hq.w4a8_int(), max_m=M, tuning=tuning)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV))
    out = plan.gemm(d["a_codes"].to(DEV), w, meta, a_scale=d["a_scale"].to(DEV))
    torch.cuda.synchronize()
    assert "kernel=tiled" in plan.describe(M)
    ref = og.gemm_int4_int8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["scales"].double().numpy())
    _assert_ok(out.double().cpu().numpy(), ref, "bf16", "tiled w4a8-int")
    # INT4 x fp8
    rng = np.random.default_rng(5)
    a_codes, a_scale = datagen.quant_per_token(torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)), "fp8")
    zeros = rng.integers(0, 16, size=(N, K // 128), dtype=np.uint8)
    plan = hq.Plan(N, K, hq.w4a8_fp8(zp="u4"), max_m=M, tuning=tuning)
    w, meta = plan.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV), torch.from_numpy(zeros).to(DEV))
    out = plan.gemm(a_codes.to(DEV), w, meta, a_scale=a_scale.to(DEV))
    torch.cuda.synchronize()
    ref = _fp8_oracle(a_codes.numpy(), a_scale.numpy(), d["codes"], d["scales"].double().numpy(), zeros)
    _assert_ok(out.double().cpu().numpy(), ref, "bf16", "tiled w4a8-fp8")
