"""C-ABI checks that need no GPU.

* The built library loads and exports every function include/hq.h declares.
* Host-side validation rejects bad descriptions, tunings and call arguments
  before any launch (every call below fails validation, so nothing reaches a
  device on any machine).
* The host repack (hq_repack_host; the device repack is checked against it
  on the GPU) produces the operand order each matrix instruction needs.  The
  requirement is restated here from the MFMA operand definitions, not from the
  library's code: lane l of the 16 x 128 fragment (nb, g) serves column
  16 nb + l % 16, and every extracted operand register must hold the codes of
  the k its activation partner in the same lane holds (16-bit step t:
  k = 32 t + 8 (l // 16) + [0, 8); 8-bit piece h: k = 64 h + 16 (l // 16) +
  [0, 16)); MXFP4 lanes hold the E8M0 block [128 g + 32 (l // 16), +32).
"""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_gemm_repack_amd as hq
import datagen
from oracle.formats import unpack_u4
from oracle.gemm import unpack_u2, unpack_u3


def _plan(n=256, k=512, quant=None, max_m=64, epi="none", tuning=None, fallback=False):
    # the C rejection path: no binding-level fallback unless asked for
    return hq.Plan(n, k, quant if quant is not None else hq.w4a16(), max_m=max_m, epi=epi, tuning=tuning,
                   fallback=fallback)


def test_library_exports_every_header_function():
    L = hq.lib()
    names = hq.header_functions()
    assert {"hq_plan_create", "hq_repack", "hq_gemm", "hq_last_error"} <= set(names)
    for name in names:
        assert hasattr(L, name), f"{name} declared in include/hq.h but not exported"


def test_library_has_no_undefined_internal_symbols():
    # every kernel launched from host code must have its host stub in the
    # library (a kernel body the host pass cannot instantiate drops the stub
    # without a diagnostic, and the library then fails to load on a GPU host)
    import subprocess
    r = subprocess.run(["nm", "-D", "--undefined-only", hq.lib()._name], capture_output=True, text=True, check=True)
    bad = [l.split()[-1] for l in r.stdout.splitlines() if "_ZN2hq" in l]
    assert not bad, f"undefined library symbols: {bad[:5]}"


def test_abi_version_and_status_strings():
    L = hq.lib()
    assert L.hq_abi_version() == 3
    assert L.hq_status_str(0) == b"HQ_OK"
    assert L.hq_status_str(3) == b"HQ_ERR_WORKSPACE"


@pytest.mark.parametrize("kw, status", [
    (dict(k=500), hq.HQ_ERR_UNSUPPORTED),          # K not a multiple of 128
    (dict(n=250), hq.HQ_ERR_UNSUPPORTED),          # N not a multiple of 16
    (dict(max_m=-1), hq.HQ_ERR_INVALID_ARG),
    (dict(quant=hq.QuantDesc(hq.U4, 3, 128, hq.F16, hq.ZP_FIXED, 8, hq.F16, 0, hq.F16)), hq.HQ_ERR_UNSUPPORTED),
    (dict(quant=hq.QuantDesc(hq.U4, 4, 64, hq.F16, hq.ZP_FIXED, 8, hq.F16, 0, hq.F16)), hq.HQ_ERR_UNSUPPORTED),
    (dict(quant=hq.QuantDesc(hq.U4, 4, 128, hq.F16, hq.ZP_FIXED, 16, hq.F16, 0, hq.F16)), hq.HQ_ERR_INVALID_ARG),
    (dict(quant=hq.QuantDesc(hq.U4, 4, 128, hq.F16, hq.ZP_PER_GROUP_U4, 0, hq.INT8, 1, hq.BF16)),
     hq.HQ_ERR_UNSUPPORTED),                       # INT4 x INT8 needs zero 8
    (dict(quant=hq.QuantDesc(hq.FP4_E2M1, 4, 32, hq.E8M0, hq.ZP_NONE, 0, hq.BF16, 0, hq.BF16)),
     hq.HQ_ERR_UNSUPPORTED),                       # MXFP4 x bf16 not implemented
    (dict(quant=hq.QuantDesc(hq.U4, 4, 128, hq.F16, hq.ZP_FIXED, 8, hq.INT8, 0, hq.BF16)),
     hq.HQ_ERR_UNSUPPORTED),                       # int8 activations without scales
    (dict(epi="i32_acc"), hq.HQ_ERR_UNSUPPORTED),  # int32 accumulators need INT4 x INT8
    (dict(tuning=dict(tile_m=48)), hq.HQ_ERR_INVALID_ARG),
    (dict(tuning=dict(kernel=1, tile_n=128)), hq.HQ_ERR_INVALID_ARG),
    (dict(tuning=dict(kernel=2, tile_n=192)), hq.HQ_ERR_INVALID_ARG),
    (dict(tuning=dict(kernel=2, split_k=65)), hq.HQ_ERR_INVALID_ARG),
    (dict(tuning=dict(kernel=1, waves=9)), hq.HQ_ERR_INVALID_ARG),
    (dict(tuning=dict(kernel=1, stages=3)), hq.HQ_ERR_INVALID_ARG),
    (dict(tuning=dict(kernel=1, tile_m=64, tile_n=64, stages=4)), hq.HQ_ERR_INVALID_ARG),  # register budget
])
def test_plan_validation(kw, status):
    with pytest.raises(hq.HQError) as e:
        _plan(**kw)
    assert e.value.status == status
    assert hq.lib().hq_last_error().decode()


NVFP4_FP8 = hq.QuantDesc(hq.FP4_E2M1, 4, 16, hq.FP8_E4M3, hq.ZP_NONE, 0, hq.FP8_E4M3, hq.ASCALE_PER_TOKEN_F32, hq.BF16)
MXINT4_FP8 = hq.QuantDesc(hq.I4, 4, 32, hq.E8M0, hq.ZP_NONE, 0, hq.FP8_E4M3, hq.ASCALE_PER_TOKEN_F32, hq.BF16)
INT4U4_I8 = hq.QuantDesc(hq.U4, 4, 128, hq.F16, hq.ZP_PER_GROUP_U4, 0, hq.INT8, hq.ASCALE_PER_TOKEN_F32, hq.F16)


def test_mfma_in_must_name_the_descriptions_type():
    for q, mi in ((hq.w4a16("bf16"), "bf16"), (hq.w4a16("f16"), "f16"), (hq.w4a8_int(), "int8"),
                  (hq.w4a8_fp8(), "fp8"), (hq.w4a8_mxfp4(), "fp8xfp4"), (hq.w4a4_mxfp4(), "fp4")):
        p = hq.Plan(4096, 4096, q, max_m=16, mfma_in=mi, fallback=False)
        assert f"mfma={mi}" in p.describe(16) and p.fallback is None
        other = "f16" if mi != "f16" else "bf16"
        with pytest.raises(hq.HQError) as e:
            hq.Plan(4096, 4096, q, max_m=16, mfma_in=other, fallback=False)
        assert e.value.status == hq.HQ_ERR_UNSUPPORTED and "matrix instruction" in str(e.value)
    # an out-of-range value through the C ABI
    L = hq.lib()
    layer = hq.LayerDesc(4096, 4096, 1, hq.w4a16())
    h = ctypes.c_void_p()
    assert L.hq_plan_create(ctypes.byref(layer), ctypes.byref(hq.Compute(0, 0, 7)), 16, None,
                            ctypes.byref(h)) == hq.HQ_ERR_INVALID_ARG


@pytest.mark.parametrize("q, runs", [(NVFP4_FP8, "w4a16-nvfp4-bf16"), (MXINT4_FP8, "w4a16-mxint4-bf16"),
                                     (INT4U4_I8, "w4a16-f16")])
def test_unsupported_compute_type_falls_back_to_16_bit_activations(q, runs):
    # the C library rejects the description ...
    with pytest.raises(hq.HQError) as e:
        hq.Plan(4096, 4096, q, max_m=64, fallback=False)
    assert e.value.status == hq.HQ_ERR_UNSUPPORTED
    # ... and the binding builds the same weights with 16-bit activations
    p = hq.Plan(4096, 4096, q, max_m=64)
    assert p.fallback and p.requested_quant is q
    assert p.quant.act == q.out and p.quant.act_scale == hq.ASCALE_NONE
    assert (p.quant.w_elem, p.quant.group_size, p.quant.scale, p.quant.zp) == (q.w_elem, q.group_size, q.scale, q.zp)
    d = p.describe(16)
    assert f"fmt={runs}" in d and "fallback=16-bit-activations" in d
    # a requested instruction type the description cannot use falls back too
    p2 = hq.Plan(4096, 4096, hq.w4a8_int(), max_m=64, mfma_in="fp8")
    assert p2.fallback and "fmt=w4a16-bf16" in p2.describe(1)


def test_fallback_never_hides_other_errors():
    with pytest.raises(hq.HQError) as e:   # invalid argument: no fallback
        hq.Plan(250, 4096, hq.w4a8_int(), max_m=64)
    assert e.value.status == hq.HQ_ERR_UNSUPPORTED and "N must be a multiple" in str(e.value)
    with pytest.raises(hq.HQError):        # no 16-bit kernel for MXFP4 weights either: the original error
        hq.Plan(4096, 4096, hq.w4a8_mxfp4(), max_m=64, mfma_in="int8")
    with pytest.raises(hq.HQError):        # 16-bit activations were asked for: nothing higher to fall to
        hq.Plan(4096, 4096, hq.w4a16("bf16"), max_m=64, mfma_in="fp8")


def test_grouped_epilogue_on_dense_plan_rejected():
    with pytest.raises(hq.HQError) as e:
        _plan(epi="silu_mul")
    assert e.value.status == hq.HQ_ERR_UNSUPPORTED


def test_null_arguments_rejected():
    L = hq.lib()
    h = ctypes.c_void_p()
    assert L.hq_plan_create(None, None, 1, None, ctypes.byref(h)) == hq.HQ_ERR_INVALID_ARG
    b = ctypes.c_size_t()
    assert L.hq_plan_workspace_bytes(None, 1, ctypes.byref(b)) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_gemm(None, 1, None, None, None, None, None, None, 0, None) == hq.HQ_ERR_INVALID_ARG


# Fake, never-dereferenced device addresses: every call below is rejected by
# validation before any launch.
_A16 = 0x10000


def _gemm_status(plan, m, a=_A16, a_scale=None, w=_A16, meta=_A16, out=_A16, ws=None, ws_bytes=0):
    return hq.lib().hq_gemm(plan._h, m, a, a_scale, w, meta, out, ws, ws_bytes, None)


def test_gemm_argument_validation():
    p = _plan(max_m=16)
    assert _gemm_status(p, 17) == hq.HQ_ERR_INVALID_ARG             # m > max_m
    assert _gemm_status(p, -1) == hq.HQ_ERR_INVALID_ARG
    assert _gemm_status(p, 0) == hq.HQ_OK                            # m = 0 is a no-op
    assert _gemm_status(p, 4, a=None) == hq.HQ_ERR_INVALID_ARG       # null
    assert _gemm_status(p, 4, w=_A16 + 4) == hq.HQ_ERR_INVALID_ARG  # misaligned
    assert _gemm_status(p, 4, a_scale=_A16) == hq.HQ_ERR_INVALID_ARG  # 16-bit A takes no scale
    p8 = _plan(quant=hq.w4a8_int(), max_m=16)
    assert _gemm_status(p8, 4) == hq.HQ_ERR_INVALID_ARG              # int8 A needs scales


def test_workspace_validation():
    # force a cross-workgroup split so that a workspace is required
    p = _plan(n=256, k=4096, max_m=16, tuning=dict(split_k=4))
    need = p.workspace_bytes(16)
    assert need > 0
    assert _gemm_status(p, 16, ws=None) == hq.HQ_ERR_WORKSPACE
    assert _gemm_status(p, 16, ws=_A16, ws_bytes=need - 1) == hq.HQ_ERR_WORKSPACE
    assert _plan(n=256, k=4096, max_m=16, tuning=dict(split_k=1)).workspace_bytes(16) == 0


def test_describe_and_sizes():
    p = _plan(n=4096, k=4096, quant=hq.w4a16("bf16", zp="u4"), max_m=64)
    s = p.describe(16)
    assert "w4a16-bf16" in s and "split_k" in s
    w, m = p.repacked_bytes()
    assert w == 4096 * 4096 // 2
    assert m == 4096 * 32 * 2 + (4096 // 16) * 32 * 8
    pm = _plan(n=4096, k=7168, quant=hq.w4a8_mxfp4(), max_m=16)
    assert pm.repacked_bytes() == (4096 * 7168 // 2, 4096 * 7168 // 32)


# ---------------------------------------------------------------- layout ----

N, K = 48, 384  # three column blocks, three groups


def _codes(seed=0):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    return q, datagen.pack_u4(q)


def _frag_words(w: np.ndarray):
    """Device bytes -> words[nb, g, lane, t]."""
    return w.view(np.uint32).reshape(N // 16, K // 128, 64, 4)


def _lane_k(g, lane):
    return 128 * g + 32 * (lane // 16)


# k of each activation-operand piece, per lane quarter kq = lane // 16:
# 16-bit MFMA step t: 32 t + 8 kq + [0, 8); 8-bit piece h: 64 h + 16 kq + [0, 16)
def _k16(g, lane, t):
    return 128 * g + 32 * t + 8 * (lane // 16)


def _k8(g, lane, h):
    return 128 * g + 64 * h + 16 * (lane // 16)


def test_repack_w16_operand_order():
    q, codes = _codes(1)
    p = _plan(N, K, hq.w4a16("f16"), max_m=16)
    w, _ = p.repack_host(torch.from_numpy(codes), torch.ones(N, K // 128, dtype=torch.float16))
    fw = _frag_words(w.numpy())
    for nb in range(N // 16):
        for g in range(K // 128):
            for lane in range(64):
                n = 16 * nb + lane % 16
                for t in range(4):
                    x = int(fw[nb, g, lane, t])
                    k0 = _k16(g, lane, t)
                    for r in range(4):  # operand register r: 16-bit halves = k-offsets 2r, 2r+1
                        v = (x >> (4 * r)) & 0x000F000F
                        assert v & 0xF == q[n, k0 + 2 * r]
                        assert v >> 16 == q[n, k0 + 2 * r + 1]


def test_repack_int8_operand_order():
    q, codes = _codes(2)
    p = _plan(N, K, hq.w4a8_int(), max_m=16)
    w, _ = p.repack_host(torch.from_numpy(codes), torch.ones(N, K // 128, dtype=torch.float16))
    fw = _frag_words(w.numpy())
    for nb in range(N // 16):
        for g in range(K // 128):
            for lane in range(64):
                n = 16 * nb + lane % 16
                for step in range(2):  # int8 MFMA 16x16x64: 16 k per lane per step
                    k0 = _k8(g, lane, step)
                    w0, w1 = int(fw[nb, g, lane, 2 * step]), int(fw[nb, g, lane, 2 * step + 1])
                    regs = [(w0 << 4) & 0xF0F0F0F0, w0 & 0xF0F0F0F0, (w1 << 4) & 0xF0F0F0F0, w1 & 0xF0F0F0F0]
                    for j, reg in enumerate(regs):
                        for b in range(4):
                            byte = (reg >> (8 * b)) & 0xFF
                            val = byte - 256 if byte >= 128 else byte
                            assert val == 16 * (int(q[n, k0 + 4 * j + b]) - 8)


def test_repack_fp8_operand_order():
    q, codes = _codes(3)
    p = _plan(N, K, hq.w4a8_fp8(), max_m=16)
    w, _ = p.repack_host(torch.from_numpy(codes), torch.ones(N, K // 128, dtype=torch.float16))
    fw = _frag_words(w.numpy())
    for nb in range(N // 16):
        for g in range(K // 128):
            for lane in range(64):
                n = 16 * nb + lane % 16
                for t in range(4):  # operand registers 2t, 2t+1 of the 8-register fp8 operand
                    x = int(fw[nb, g, lane, t])
                    k0 = _k8(g, lane, t // 2) + 8 * (t % 2)
                    for h, reg in enumerate((x & 0x0F0F0F0F, (x >> 4) & 0x0F0F0F0F)):
                        for b in range(4):
                            assert (reg >> (8 * b)) & 0xFF == q[n, k0 + 4 * h + b]


def test_repack_mxfp4_operand_order_and_e8m0():
    q, codes = _codes(4)
    rng = np.random.default_rng(5)
    e8 = rng.integers(119, 124, size=(N, K // 32), dtype=np.uint8)
    p = _plan(N, K, hq.w4a8_mxfp4(), max_m=16)
    w, meta = p.repack_host(torch.from_numpy(codes), e8m0=torch.from_numpy(e8))
    wb = w.numpy().reshape(N // 16, K // 128, 64, 16)
    mb = meta.numpy().reshape(N // 16, K // 128, 64)
    for nb in range(N // 16):
        for g in range(K // 128):
            for lane in range(64):
                n, k0 = 16 * nb + lane % 16, _lane_k(g, lane)
                nib = np.stack([wb[nb, g, lane] & 0xF, wb[nb, g, lane] >> 4], axis=1).reshape(-1)
                assert np.array_equal(nib, q[n, k0:k0 + 32])  # element j: byte j/2, low nibble first
                assert mb[nb, g, lane] == e8[n, k0 // 32]


def test_repack_scales_and_zeros():
    q, codes = _codes(6)
    rng = np.random.default_rng(7)
    scales = torch.from_numpy(rng.uniform(0.005, 0.02, size=(N, K // 128))).to(torch.bfloat16)
    zeros = rng.integers(0, 16, size=(N, K // 128), dtype=np.uint8)
    p = _plan(N, K, hq.w4a16("bf16", zp="u4"), max_m=16)
    w, meta = p.repack_host(torch.from_numpy(codes), scales, torch.from_numpy(zeros))
    G = K // 128
    sreg = meta[: N * G * 2].view(torch.bfloat16).reshape(N // 16, G, 16)
    zreg = meta[N * G * 2:].numpy().view(np.uint32).reshape(N // 16, G, 2)
    for nb in range(N // 16):
        for g in range(G):
            for c in range(16):
                n = 16 * nb + c
                assert sreg[nb, g, c].item() == scales[n, g].item()
                assert (int(zreg[nb, g, c // 8]) >> (4 * (c % 8))) & 0xF == zeros[n, g]


def test_repack_is_a_bijection_on_codes():
    # every canonical nibble appears exactly once in the device layout
    for quant in (hq.w4a16("f16"), hq.w4a8_fp8(), hq.w4a8_mxfp4()):
        q = np.zeros((N, K), dtype=np.uint8)
        p = _plan(N, K, quant, max_m=16)
        for bit in range(4):
            q[:] = 0
            rng = np.random.default_rng(bit)
            q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
            codes = torch.from_numpy(datagen.pack_u4(q))
            kw = dict(e8m0=torch.zeros(N, K // 32, dtype=torch.uint8)) if quant.w_elem == hq.FP4_E2M1 else \
                dict(scales=torch.ones(N, K // 128, dtype=torch.float16))
            w, _ = p.repack_host(codes, **kw)
            dev = unpack_u4(w.numpy().view(np.int32).reshape(1, -1))[0]
            assert np.array_equal(np.bincount(dev, minlength=16), np.bincount(q.reshape(-1), minlength=16))


# ------------------------------------------------------------------- MoE ----

def test_moe_plan_validation():
    with pytest.raises(hq.HQError) as e:   # grouped + INT4 x INT8 not implemented
        hq.MoePlan(512, 7168, hq.w4a8_int(), 256, 64, "silu_mul")
    assert e.value.status == hq.HQ_ERR_UNSUPPORTED
    with pytest.raises(hq.HQError) as e:   # gate + up must pair 16-column blocks
        hq.MoePlan(48, 256, hq.w4a16("bf16"), 4, 64, "silu_mul")
    assert e.value.status == hq.HQ_ERR_UNSUPPORTED
    with pytest.raises(hq.HQError):         # combine epilogue on a dense plan
        hq.Plan(512, 256, hq.w4a16("bf16"), max_m=4, epi="topk_combine")
    p = hq.MoePlan(512, 7168, hq.w4a16("bf16", scale="f16"), 256, 64, "silu_mul")
    assert p.block_m(32, 8) == 16
    assert p.repacked_bytes() == (256 * 512 * 7168 // 2, 256 * 512 * 56 * 2)


def test_moe_block_choice():
    """Host logic: the block size follows the slots per expert, or the tuning."""
    q = hq.w4a16("bf16", scale="f16")
    p = hq.MoePlan(512, 7168, q, 256, 1 << 16, "silu_mul")
    assert p.block_m(1, 8) == 16         # 0.03 slots per expert: weight streaming
    assert p.block_m(32, 8) == 16        # 1 per expert
    assert p.block_m(256, 8) == 16       # 8 per expert
    assert p.block_m(512, 8) == 64       # 16 per expert: MFMA tiles
    assert p.block_m(4096, 8) == 64      # 128 per expert: MFMA tiles
    assert p.block_m(16384, 8) == 128    # 512 per expert
    assert hq.MoePlan(512, 7168, q, 256, 64, "silu_mul", tuning=dict(tile_m=128)).block_m(1, 8) == 128
    assert hq.MoePlan(512, 7168, q, 256, 64, "silu_mul", tuning=dict(kernel=2)).block_m(1, 8) == 64
    assert hq.MoePlan(512, 7168, q, 256, 8192, "silu_mul", tuning=dict(kernel=1)).block_m(4096, 8) == 16
    assert hq.MoePlan(512, 7168, q, 256, 8192, "silu_mul", tuning=dict(tile_m=32)).block_m(4096, 8) == 32
    for bad in (dict(tile_m=48), dict(kernel=1, tile_m=64), dict(kernel=2, tile_m=32), dict(tile_n=96),
                dict(tile_n=256, tile_m=64), dict(waves=17)):
        n = 384 if bad.get("tile_n") == 256 else 512
        with pytest.raises(hq.HQError) as e:
            hq.MoePlan(n, 7168, q, 256, 64, "silu_mul", tuning=bad)
        assert e.value.status == hq.HQ_ERR_UNSUPPORTED, bad
    # the description names the kernel the grouped call launches
    assert "kernel=grouped-skinny" in p.describe(32, 8) and "block_m=16" in p.describe(32, 8)
    assert "kernel=grouped-tiled" in p.describe(4096, 8) and "block_m=64" in p.describe(4096, 8)
    down = hq.MoePlan(7168, 256, q, 256, 8192, "topk_combine")
    assert "kernel=grouped-smallk" in down.describe(32, 8) and "kernel=grouped-smallk" in down.describe(4096, 8)
    assert "kernel=grouped-tiled" in hq.MoePlan(7168, 256, q, 256, 8192, "topk_combine",
                                                tuning=dict(kernel=2)).describe(4096, 8)
    # the workspace follows the block size of the call
    pq = hq.MoePlan(512, 7168, hq.w4a8_fp8(), 256, 8192, "silu_mul_qfp8")
    b = ctypes.c_size_t()
    assert hq.lib().hq_moe_workspace_bytes(pq._h, 4096, 8, ctypes.byref(b)) == 0
    assert b.value >= hq.moe_max_padded(4096, 8, 256, 64) * 256 * 4


def test_moe_sizes_and_workspace():
    # every expert's segment + the out-of-range segment, padded, rounded up to 16
    assert hq.moe_max_padded(1, 8, 256, 16) == 8 + 257 * 15 + 9
    assert hq.moe_max_padded(4096, 8, 256, 16) == 32768 + 257 * 15 + 1
    assert hq.moe_max_padded(4096, 8, 256, 64) == 32768 + 257 * 63 + 1
    pq = hq.MoePlan(512, 7168, hq.w4a8_fp8(), 256, 4096, "silu_mul_qfp8")
    b = ctypes.c_size_t()
    assert hq.lib().hq_moe_workspace_bytes(pq._h, 32, 8, ctypes.byref(b)) == 0
    mp = hq.moe_max_padded(32, 8, 256, 16)
    assert b.value >= mp * 256 * 4
    pc = hq.MoePlan(7168, 256, hq.w4a16("bf16", scale="f16"), 256, 4096, "topk_combine")
    # the combine's weighted slot rows: t * topk rows of n bf16
    assert hq.lib().hq_moe_workspace_bytes(pc._h, 32, 8, ctypes.byref(b)) == 0 and b.value >= 32 * 8 * 7168 * 2
    assert b.value < 32 * 8 * 7168 * 2 + 256


def test_moe_call_validation():
    L = hq.lib()
    A = 0x10000
    assert L.hq_moe_align(0, 8, 256, 16, A, A, A, A, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_moe_align(4, 8, 256, 10, A, A, A, A, None) == hq.HQ_ERR_INVALID_ARG   # block_m % 16
    assert L.hq_moe_align(4, 8, 256, 16, None, A, A, A, None) == hq.HQ_ERR_INVALID_ARG
    p = hq.MoePlan(7168, 256, hq.w4a16("bf16", scale="f16"), 256, 64, "topk_combine")
    # pointer arguments: a, a_scale, sorted_ids, block_expert, num_padded, topk_w, w, meta, out, out_scale, ws
    def args(**kw):
        names = ["a", "a_scale", "sorted_ids", "block_expert", "num_padded", "topk_w", "w", "meta", "out",
                 "out_scale", "ws"]
        d = {n: A for n in names}
        d["a_scale"] = None
        d["out_scale"] = None
        d.update(kw)
        return [d[n] for n in names]
    assert L.hq_moe_gemm(p._h, 4, 8, *args(topk_w=None), 1 << 30, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_moe_gemm(p._h, 4, 8, *args(a_scale=A), 1 << 30, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_moe_gemm(p._h, 4, 8, *args(), 16, None) == hq.HQ_ERR_WORKSPACE   # workspace too small
    assert L.hq_moe_gemm(p._h, 4, 8, *args(ws=None), 1 << 30, None) == hq.HQ_ERR_WORKSPACE
    assert L.hq_moe_gemm(p._h, 65, 8, *args(), 1 << 30, None) == hq.HQ_ERR_INVALID_ARG  # t > max_t
    assert L.hq_moe_gemm(p._h, 4, 8, *args(w=A + 8), 1 << 30, None) == hq.HQ_ERR_INVALID_ARG  # misaligned
    pq = hq.MoePlan(512, 7168, hq.w4a8_fp8(), 256, 64, "silu_mul_qfp8")
    assert L.hq_moe_gemm(pq._h, 4, 8, *args(a_scale=A), 1 << 30, None) == hq.HQ_ERR_INVALID_ARG  # no out_scale


def test_moe_by_slot_call_validation():
    """Argument checks of hq_moe_gemm_by_slot run before any launch (no GPU needed)."""
    L = hq.lib()
    A = 0x10000
    p = hq.MoePlan(7168, 256, hq.w4a16("bf16", scale="f16"), 256, 64, "topk_combine")
    # pointer arguments: a, a_scale, topk_ids, topk_w, w, meta, out, out_scale, ws
    def args(**kw):
        names = ["a", "a_scale", "topk_ids", "topk_w", "w", "meta", "out", "out_scale", "ws"]
        d = {n: A for n in names}
        d["a_scale"] = d["out_scale"] = d["ws"] = None
        d.update(kw)
        return [d[n] for n in names]
    f = L.hq_moe_gemm_by_slot
    assert f(None, 1, 8, *args(), 0, None) == hq.HQ_ERR_INVALID_ARG
    assert f(p._h, 0, 8, *args(a=None), 0, None) == hq.HQ_OK                    # t = 0: nothing to do
    assert f(p._h, 1, 8, *args(topk_w=None), 0, None) == hq.HQ_ERR_INVALID_ARG   # the combine needs weights
    assert f(p._h, 1, 8, *args(topk_ids=None), 0, None) == hq.HQ_ERR_INVALID_ARG
    assert f(p._h, 1, 8, *args(a_scale=A), 0, None) == hq.HQ_ERR_INVALID_ARG     # 16-bit rows take no scale
    assert f(p._h, 65, 8, *args(), 0, None) == hq.HQ_ERR_INVALID_ARG             # t > max_t
    assert f(p._h, 1, 0, *args(), 0, None) == hq.HQ_ERR_INVALID_ARG              # topk
    assert f(p._h, 1, 65, *args(), 0, None) == hq.HQ_ERR_INVALID_ARG
    assert f(p._h, 1, 8, *args(out=A + 8), 0, None) == hq.HQ_ERR_INVALID_ARG     # misaligned
    big = hq.MoePlan(7168, 256, hq.w4a16("bf16", scale="f16"), 256, 1 << 14, "topk_combine")
    assert f(big._h, 1 << 14, 8, *args(), 0, None) == hq.HQ_ERR_UNSUPPORTED     # t * topk > 65535
    dense = hq.Plan(512, 256, hq.w4a16("bf16"), max_m=4)
    assert f(dense._h, 1, 8, *args(), 0, None) == hq.HQ_ERR_INVALID_ARG
    pq = hq.MoePlan(512, 7168, hq.w4a8_fp8(), 256, 64, "silu_mul_qfp8")
    need = 4 * 8 * 256 * 4                                                       # t * topk rows of n/2 fp32
    assert f(pq._h, 4, 8, *args(a_scale=None, out_scale=A, ws=A), need, None) == hq.HQ_ERR_INVALID_ARG
    assert f(pq._h, 4, 8, *args(a_scale=A, out_scale=None, ws=A), need, None) == hq.HQ_ERR_INVALID_ARG
    assert f(pq._h, 4, 8, *args(a_scale=A, out_scale=A, ws=None), need, None) == hq.HQ_ERR_WORKSPACE
    assert f(pq._h, 4, 8, *args(a_scale=A, out_scale=A, ws=A), need - 1, None) == hq.HQ_ERR_WORKSPACE
    # the aligned path's workspace is always enough for the same t and topk
    b = ctypes.c_size_t()
    assert L.hq_moe_workspace_bytes(pq._h, 4, 8, ctypes.byref(b)) == 0 and b.value >= need
    # all experts' weights in one buffer range (down mode): 2 GiB or more is refused
    huge = hq.MoePlan(8192, 2048, hq.w4a16("bf16", scale="f16"), 512, 64, "topk_combine")
    assert f(huge._h, 1, 8, *args(), 0, None) == hq.HQ_ERR_UNSUPPORTED


def test_moe_layer_path_choice():
    """Host logic: moe_layer takes the by-slot path up to 128 routed slots (96
    with fp8 activations)."""
    assert hq.moe_uses_by_slot(1, 8) and hq.moe_uses_by_slot(16, 8) and hq.moe_uses_by_slot(64, 2)
    assert not hq.moe_uses_by_slot(17, 8) and not hq.moe_uses_by_slot(4096, 8) and not hq.moe_uses_by_slot(0, 8)
    assert hq.moe_uses_by_slot(12, 8, fp8=True) and not hq.moe_uses_by_slot(13, 8, fp8=True)
    q = hq.w4a16("bf16", scale="f16")
    g = hq.MoePlan(512, 7168, q, 256, 64, "silu_mul")
    d = hq.MoePlan(7168, 256, q, 256, 64, "topk_combine")
    ids = torch.zeros((1, 8), dtype=torch.int32)
    with pytest.raises(ValueError):                       # plans in the wrong roles
        hq.moe_layer(d, g, None, ids, None, None, None, None, None)


def test_quantize_call_validation():
    """Argument checks of hq_quantize_per_token run before any launch (no GPU needed)."""
    L = hq.lib()
    fake = 1 << 20  # 16-byte aligned address that is never dereferenced: every call below is rejected
    q = L.hq_quantize_per_token
    assert q(4, 64, hq.F32, hq.FP8_E4M3, fake, fake, fake, None) == hq.HQ_ERR_UNSUPPORTED
    assert q(4, 64, hq.BF16, hq.BF16, fake, fake, fake, None) == hq.HQ_ERR_UNSUPPORTED
    assert q(-1, 64, hq.BF16, hq.INT8, fake, fake, fake, None) == hq.HQ_ERR_INVALID_ARG
    assert q((1 << 24) + 1, 64, hq.BF16, hq.INT8, fake, fake, fake, None) == hq.HQ_ERR_INVALID_ARG
    for k in (0, 4, 12, (1 << 24) + 8):
        assert q(4, k, hq.BF16, hq.INT8, fake, fake, fake, None) == hq.HQ_ERR_INVALID_ARG
    assert q(4, 64, hq.F16, hq.FP8_E4M3, None, fake, fake, None) == hq.HQ_ERR_INVALID_ARG
    assert q(4, 64, hq.F16, hq.FP8_E4M3, fake, None, fake, None) == hq.HQ_ERR_INVALID_ARG
    assert q(4, 64, hq.F16, hq.FP8_E4M3, fake, fake, None, None) == hq.HQ_ERR_INVALID_ARG
    assert q(4, 64, hq.F16, hq.FP8_E4M3, fake + 8, fake, fake, None) == hq.HQ_ERR_INVALID_ARG
    assert b"aligned" in L.hq_last_error()
    assert q(0, 64, hq.F16, hq.FP8_E4M3, None, None, None, None) == hq.HQ_OK  # m = 0: no-op


def test_w4a4_plans_and_validation():
    p = _plan(quant=hq.w4a4_mxfp4(), n=4096, k=7168, max_m=1024)
    assert "w4a4-mxfp4" in p.describe(1) and "kernel=skinny" in p.describe(1)
    assert "kernel=tiled" in p.describe(1024)
    for m in (1, 64, 1024):
        assert p.workspace_bytes(m) >= 0
    with pytest.raises(hq.HQError):   # W4A4 is dense only
        hq.MoePlan(512, 7168, hq.w4a4_mxfp4(), 256, 4096, "silu_mul")
    bad = hq.QuantDesc(hq.FP4_E2M1, 4, 32, hq.E8M0, hq.ZP_NONE, 0, hq.FP4_E2M1, hq.ASCALE_PER_TOKEN_F32, hq.BF16)
    with pytest.raises(hq.HQError):   # MXFP4 activations need E8M0 block scales
        _plan(quant=bad)
    # activations need their E8M0 scales
    assert _gemm_status(p, 4, a_scale=None) == hq.HQ_ERR_INVALID_ARG
    assert _gemm_status(p, 4, a_scale=_A16 + 4) == hq.HQ_ERR_INVALID_ARG


def test_quantize_mxfp4_call_validation():
    L = hq.lib()
    fake = 1 << 20
    q = L.hq_quantize_mxfp4
    assert q(4, 128, hq.F32, fake, fake, fake, None) == hq.HQ_ERR_UNSUPPORTED
    for k in (0, 16, 32, 96, 640 + 32, (1 << 24) + 128):
        assert q(4, k, hq.BF16, fake, fake, fake, None) == hq.HQ_ERR_INVALID_ARG
    assert q(-1, 128, hq.BF16, fake, fake, fake, None) == hq.HQ_ERR_INVALID_ARG
    assert q(1 << 24, 1 << 13, hq.BF16, fake, fake, fake, None) == hq.HQ_ERR_UNSUPPORTED  # m * k above 2^36
    assert q(4, 128, hq.BF16, None, fake, fake, None) == hq.HQ_ERR_INVALID_ARG
    assert q(4, 128, hq.BF16, fake, fake, fake + 1, None) == hq.HQ_ERR_INVALID_ARG
    assert q(0, 128, hq.BF16, None, None, None, None) == hq.HQ_OK


def test_repack_w8_planes_operand_order():
    """INT8 weights: per fragment a high-nibble plane then a low-nibble plane,
    each in the 16-bit operand order, so 16 * high + low is the code."""
    rng = np.random.default_rng(9)
    q = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    p = _plan(N, K, hq.w8a16("f16"), max_m=16)
    w, _ = p.repack_host(torch.from_numpy(q), torch.ones(N, K // 128, dtype=torch.float16))
    fw = w.numpy().view(np.uint32).reshape(N // 16, K // 128, 2, 64, 4)
    for nb in range(N // 16):
        for g in range(K // 128):
            for lane in range(0, 64, 5):
                n = 16 * nb + lane % 16
                for t in range(4):
                    k0 = _k16(g, lane, t)
                    for r in range(4):
                        hi = (int(fw[nb, g, 0, lane, t]) >> (4 * r)) & 0x000F000F
                        lo = (int(fw[nb, g, 1, lane, t]) >> (4 * r)) & 0x000F000F
                        assert 16 * (hi & 0xF) + (lo & 0xF) == q[n, k0 + 2 * r]
                        assert 16 * (hi >> 16) + (lo >> 16) == q[n, k0 + 2 * r + 1]


def test_w8a16_plans_and_validation():
    p = _plan(4096, 4096, hq.w8a16("bf16"), max_m=1024)
    wb, mb = p.repacked_bytes()
    assert wb == 4096 * 4096 and mb == 4096 * 32 * 2
    assert "w8a16-bf16" in p.describe(1) and "kernel=tiled" in p.describe(1024)
    with pytest.raises(hq.HQError):   # INT8 weights take a fixed zero point only
        _plan(quant=hq.QuantDesc(hq.U8, 8, 128, hq.F16, hq.ZP_PER_GROUP_U4, 0, hq.F16, 0, hq.F16))
    with pytest.raises(hq.HQError):   # zero point range
        _plan(quant=hq.w8a16("f16", zp_value=256))
    with pytest.raises(hq.HQError):   # dense only
        hq.MoePlan(512, 7168, hq.w8a16("bf16"), 256, 4096, "silu_mul")
    with pytest.raises(hq.HQError):   # U4 elements need w_bits 4
        _plan(quant=hq.QuantDesc(hq.U4, 8, 128, hq.F16, hq.ZP_FIXED, 8, hq.F16, 0, hq.F16))


def test_repack_w2_operand_order():
    """INT2 weights: 512-byte fragments, two words per lane; word d holds MFMA
    steps 2d and 2d + 1, and (word >> 2 (4u + r)) & 0x00030003 is operand
    register r of step 2d + u (elements 2r and 2r + 1 of the lane's 8)."""
    rng = np.random.default_rng(10)
    words = rng.integers(0, 1 << 32, size=(N, K // 16), dtype=np.uint64).astype(np.uint32).view(np.int32)
    q = unpack_u2(words)
    p = _plan(N, K, hq.w2a16("f16"), max_m=16)
    w, _ = p.repack_host(torch.from_numpy(words), torch.ones(N, K // 128, dtype=torch.float16))
    assert w.numel() == N * K // 4
    fw = w.numpy().view(np.uint32).reshape(N // 16, K // 128, 64, 2)
    for nb in range(N // 16):
        for g in range(K // 128):
            for lane in range(0, 64, 3):
                n = 16 * nb + lane % 16
                for t in range(4):
                    k0 = _k16(g, lane, t)
                    y = int(fw[nb, g, lane, t >> 1]) >> (8 * (t & 1))
                    for r in range(4):
                        v = (y >> (2 * r)) & 0x00030003
                        assert (v & 0x3) == q[n, k0 + 2 * r]
                        assert (v >> 16) == q[n, k0 + 2 * r + 1]


def test_w2a16_plans_and_validation():
    p = _plan(4096, 4096, hq.w2a16("bf16"), max_m=1024)
    wb, mb = p.repacked_bytes()
    assert wb == 4096 * 4096 // 4 and mb == 4096 * 32 * 2
    assert "w2a16-bf16" in p.describe(1) and "kernel=tiled" in p.describe(1024)
    with pytest.raises(hq.HQError):   # fixed zero point only
        _plan(quant=hq.QuantDesc(hq.U2, 2, 128, hq.F16, hq.ZP_PER_GROUP_U4, 0, hq.F16, 0, hq.F16))
    with pytest.raises(hq.HQError):   # zero point range
        _plan(quant=hq.w2a16("f16", zp_value=4))
    with pytest.raises(hq.HQError):   # group 128 only
        _plan(quant=hq.QuantDesc(hq.U2, 2, 64, hq.F16, hq.ZP_FIXED, 2, hq.F16, 0, hq.F16))
    with pytest.raises(hq.HQError):   # U2 elements need w_bits 2
        _plan(quant=hq.QuantDesc(hq.U2, 4, 128, hq.F16, hq.ZP_FIXED, 2, hq.F16, 0, hq.F16))
    with pytest.raises(hq.HQError):   # dense only
        hq.MoePlan(512, 7168, hq.w2a16("bf16"), 256, 4096, "silu_mul")


def test_repack_w3_planes_operand_order():
    """INT3 weights: 768-byte fragments, the low two bits of every code in the
    INT2 layout (two words per lane) then the high bit, one word per lane,
    with (word >> (4t + r)) & 0x00010001 the high bits of operand register r
    of step t; 4 * high + low is the code of the canonical bit stream."""
    rng = np.random.default_rng(11)
    words = rng.integers(0, 1 << 32, size=(N, K // 32 * 3), dtype=np.uint64).astype(np.uint32).view(np.int32)
    q = unpack_u3(words)
    p = _plan(N, K, hq.w3a16("bf16"), max_m=16)
    w, _ = p.repack_host(torch.from_numpy(words), torch.ones(N, K // 128, dtype=torch.bfloat16))
    assert w.numel() == N * K * 3 // 8
    fw = w.numpy().view(np.uint32).reshape(N // 16, K // 128, 192)
    for nb in range(N // 16):
        for g in range(K // 128):
            for lane in range(0, 64, 3):
                n = 16 * nb + lane % 16
                hw = int(fw[nb, g, 128 + lane])
                for t in range(4):
                    k0 = _k16(g, lane, t)
                    y = int(fw[nb, g, 2 * lane + (t >> 1)]) >> (8 * (t & 1))
                    for r in range(4):
                        lo = (y >> (2 * r)) & 0x00030003
                        hi = (hw >> (4 * t + r)) & 0x00010001
                        assert 4 * (hi & 1) + (lo & 3) == q[n, k0 + 2 * r]
                        assert 4 * (hi >> 16) + (lo >> 16) == q[n, k0 + 2 * r + 1]


def test_w3a16_plans_and_validation():
    p = _plan(4096, 4096, hq.w3a16("f16"), max_m=1024)
    wb, mb = p.repacked_bytes()
    assert wb == 4096 * 4096 * 3 // 8 and mb == 4096 * 32 * 2
    assert "w3a16-f16" in p.describe(1) and "kernel=tiled" in p.describe(1024)
    with pytest.raises(hq.HQError):   # fixed zero point only
        _plan(quant=hq.QuantDesc(hq.U3, 3, 128, hq.F16, hq.ZP_PER_GROUP_U4, 0, hq.F16, 0, hq.F16))
    with pytest.raises(hq.HQError):   # zero point range
        _plan(quant=hq.w3a16("f16", zp_value=8))
    with pytest.raises(hq.HQError):   # U3 elements need w_bits 3
        _plan(quant=hq.QuantDesc(hq.U3, 2, 128, hq.F16, hq.ZP_FIXED, 4, hq.F16, 0, hq.F16))
    with pytest.raises(hq.HQError):   # dense only
        hq.MoePlan(512, 7168, hq.w3a16("bf16"), 256, 4096, "silu_mul")


def test_per_m_tuning_table():
    """hq_plan_set_tuning / hq_plan_get_tuning: an entry replaces the heuristic
    for exactly its m (describe and workspace follow it), None removes it."""
    p = _plan(4096, 4096, hq.w4a16("bf16"), max_m=1024)
    heur, tuned = p.get_tuning(1)
    assert not tuned and heur["kernel"] == 1
    t = dict(kernel=1, tile_m=16, tile_n=32, waves=4, split_k=2, stages=4)
    p.set_tuning(1, t)
    got, tuned = p.get_tuning(1)
    assert tuned and got == dict(t, tile_group=0)   # no launch-order groups on the skinny kernel
    d = p.describe(1)
    assert "tile_n=32 waves=4 split_k=2 stages=4" in d
    assert p.workspace_bytes(1) == 2 * 1 * 4096 * 4
    assert p.get_tuning(2) == (heur, False)          # other m keep the heuristic
    p.set_tuning(300, dict(kernel=2, tile_m=128, tile_n=256, stages=2, split_k=1))
    assert p.get_tuning(300) == (dict(kernel=2, tile_m=128, tile_n=256, waves=4, split_k=1, stages=2, tile_group=8),
                                 True)
    p.set_tuning(1, None)
    assert p.get_tuning(1) == (heur, False)
    with pytest.raises(hq.HQError):   # not a tile width
        p.set_tuning(4, dict(kernel=1, tile_n=48))
    with pytest.raises(hq.HQError):   # m out of range
        p.set_tuning(1025, t)
    with pytest.raises(hq.HQError):   # grouped plans keep their own choice
        hq.MoePlan(512, 7168, hq.w4a16("bf16"), 256, 4096, "silu_mul").set_tuning(1, t)


def test_autotune_argument_checks():
    """Rejected before any device work (no GPU needed)."""
    L = hq.lib()
    p = _plan(256, 512, hq.w4a16("f16"), max_m=64)
    fake = 1 << 20
    at = L.hq_plan_autotune
    assert at(p._h, 1, fake, None, fake, fake, fake, None, 0, 0, 0, None, None) == hq.HQ_ERR_INVALID_ARG  # reps
    assert at(p._h, 1, fake, None, fake, fake, fake, None, 0, 5, 8, None, None) == hq.HQ_ERR_INVALID_ARG  # flush
    assert at(p._h, 0, fake, None, fake, fake, fake, None, 0, 5, 0, None, None) == hq.HQ_ERR_INVALID_ARG  # m
    assert at(p._h, 65, fake, None, fake, fake, fake, None, 0, 5, 0, None, None) == hq.HQ_ERR_INVALID_ARG
    assert at(p._h, 1, None, None, fake, fake, fake, None, 0, 5, 0, None, None) == hq.HQ_ERR_INVALID_ARG
    assert at(p._h, 1, fake, fake, fake, fake, fake, None, 0, 5, 0, None, None) == hq.HQ_ERR_INVALID_ARG  # a_scale
    assert at(None, 1, fake, None, fake, fake, fake, None, 0, 5, 0, None, None) == hq.HQ_ERR_INVALID_ARG


def test_repack_mxint4_layout():
    """MXINT4: codes in the 16-bit operand order stored as q xor 8 (offset
    binary), and one E8M0 dword per column per fragment holding the scales of
    its four 32-k blocks (byte t = block 4g + t)."""
    rng = np.random.default_rng(12)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    e8 = rng.integers(0, 256, size=(N, K // 32), dtype=np.uint8)
    p = _plan(N, K, hq.w4a16_mxint4("bf16"), max_m=16)
    w, meta = p.repack_host(torch.from_numpy(datagen.pack_u4(q)), e8m0=torch.from_numpy(e8))
    assert meta.numel() == N * K // 32
    fw = w.numpy().view(np.uint32).reshape(N // 16, K // 128, 64, 4)
    fm = meta.numpy().reshape(N // 16, K // 128, 16, 4)
    for nb in range(N // 16):
        for g in range(K // 128):
            assert np.array_equal(fm[nb, g], e8[16 * nb:16 * nb + 16, 4 * g:4 * g + 4])
            for lane in range(0, 64, 7):
                n = 16 * nb + lane % 16
                for t in range(4):
                    k0 = _k16(g, lane, t)
                    for r in range(4):
                        v = (int(fw[nb, g, lane, t]) >> (4 * r)) & 0x000F000F
                        assert (v & 0xF) == q[n, k0 + 2 * r] ^ 8
                        assert (v >> 16) == q[n, k0 + 2 * r + 1] ^ 8


def test_mxint4_plans_and_validation():
    p = _plan(4096, 4096, hq.w4a16_mxint4("f16"), max_m=1024)
    wb, mb = p.repacked_bytes()
    assert wb == 4096 * 4096 // 2 and mb == 4096 * 4096 // 32
    assert "w4a16-mxint4-f16" in p.describe(1) and "kernel=tiled" in p.describe(1024)
    with pytest.raises(hq.HQError):   # block 32 only
        _plan(quant=hq.QuantDesc(hq.I4, 4, 128, hq.E8M0, hq.ZP_NONE, 0, hq.BF16, 0, hq.BF16))
    with pytest.raises(hq.HQError):   # E8M0 scales only
        _plan(quant=hq.QuantDesc(hq.I4, 4, 32, hq.BF16, hq.ZP_NONE, 0, hq.BF16, 0, hq.BF16))
    with pytest.raises(hq.HQError):   # 16-bit activations only
        _plan(quant=hq.QuantDesc(hq.I4, 4, 32, hq.E8M0, hq.ZP_NONE, 0, hq.FP8_E4M3, 1, hq.BF16))
    with pytest.raises(hq.HQError):   # dense only
        hq.MoePlan(512, 7168, hq.w4a16_mxint4("bf16"), 256, 4096, "silu_mul")


def test_repack_nvfp4_layout():
    """NVFP4: E2M1 codes in the 16-bit operand order (unchanged), the E4M3
    scales as [N/16][G][16 columns][2 halves][4 steps] bytes (byte t of half h
    = block 8g + 2t + h) and the fp32 tensor scale after them."""
    rng = np.random.default_rng(13)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    e4 = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    p = _plan(N, K, hq.w4a16_nvfp4("bf16"), max_m=16)
    w, meta = p.repack_host(torch.from_numpy(datagen.pack_u4(q)), torch.tensor([0.375], dtype=torch.float32),
                            e8m0=torch.from_numpy(e4))
    assert meta.numel() == N * K // 16 + 16
    fm = meta.numpy()[:N * K // 16].reshape(N // 16, K // 128, 16, 2, 4)
    assert meta.numpy()[N * K // 16:N * K // 16 + 4].view(np.float32)[0] == 0.375
    fw = w.numpy().view(np.uint32).reshape(N // 16, K // 128, 64, 4)
    for nb in range(N // 16):
        for g in range(K // 128):
            for c in range(16):
                for h in range(2):
                    for t in range(4):
                        assert fm[nb, g, c, h, t] == e4[16 * nb + c, 8 * g + 2 * t + h]
            for lane in range(0, 64, 7):
                n = 16 * nb + lane % 16
                for t in range(4):
                    k0 = _k16(g, lane, t)
                    assert (k0 % 128) // 16 == 2 * t + (lane // 16) // 2   # the lane's 8 k in one block
                    for r in range(4):
                        v = (int(fw[nb, g, lane, t]) >> (4 * r)) & 0x000F000F
                        assert (v & 0xF) == q[n, k0 + 2 * r] and (v >> 16) == q[n, k0 + 2 * r + 1]


def test_nvfp4_plans_and_validation():
    p = _plan(4096, 4096, hq.w4a16_nvfp4("f16"), max_m=1024)
    wb, mb = p.repacked_bytes()
    assert wb == 4096 * 4096 // 2 and mb == 4096 * 4096 // 16 + 16
    assert "w4a16-nvfp4-f16" in p.describe(1) and "kernel=tiled" in p.describe(1024)
    with pytest.raises(hq.HQError):   # block 16 only
        _plan(quant=hq.QuantDesc(hq.FP4_E2M1, 4, 32, hq.FP8_E4M3, hq.ZP_NONE, 0, hq.BF16, 0, hq.BF16))
    with pytest.raises(hq.HQError):   # 16-bit activations only
        _plan(quant=hq.QuantDesc(hq.FP4_E2M1, 4, 16, hq.FP8_E4M3, hq.ZP_NONE, 0, hq.FP8_E4M3, 1, hq.BF16))
    with pytest.raises(hq.HQError):   # dense only
        hq.MoePlan(512, 7168, hq.w4a16_nvfp4("bf16"), 256, 4096, "silu_mul")
    L = hq.lib()
    fake = 1 << 20
    assert L.hq_repack_host(p._h, fake, None, fake, fake, fake) == hq.HQ_ERR_INVALID_ARG   # no tensor scale


def test_mfma_probe_validation():
    # argument checks happen before any launch (no GPU needed)
    L = hq.lib()
    fake = ctypes.c_void_p(256)
    fl = ctypes.c_double()
    for kind, wg, it in ((-1, 1, 1), (6, 1, 1), (0, 0, 1), (0, 1 << 21, 1), (0, 1, 0), (0, 1, (1 << 24) + 1)):
        assert L.hq_mfma_peak(kind, wg, it, fake, ctypes.byref(fl), None) == hq.HQ_ERR_INVALID_ARG, (kind, wg, it)
    assert L.hq_mfma_peak(0, 1, 1, None, ctypes.byref(fl), None) == hq.HQ_ERR_INVALID_ARG



def test_tile_group_choice_and_validation():
    """The tiled kernel's launch order: groups of tile_group row tiles walked
    column by column (8 unless a tuning says otherwise), 1..64."""
    p = _plan(quant=hq.w4a8_mxfp4(), n=4096, k=7168, max_m=1024)
    assert "tile_group=8" in p.describe(1024) and p.get_tuning(1024)[0]["tile_group"] == 8
    q = _plan(quant=hq.w4a16("f16"), n=512, k=1024, max_m=256, tuning=dict(kernel=2, tile_group=3))
    assert "tile_group=3" in q.describe(256)
    for bad in (-1, 65):
        with pytest.raises(hq.HQError):
            _plan(quant=hq.w4a16("f16"), n=512, k=1024, max_m=256, tuning=dict(kernel=2, tile_group=bad))
