"""MoE parity on the GPU: hq_moe_align, the grouped gate_up (+ SiLU * mul, or
+ per-row fp8 requant) and the grouped down + top-k combine, each checked on
the GPU's own input to that stage against the CPU oracle (oracle/moe.py).

Layer: one GPU's tensor-parallel share of a DeepSeek-style layer -- 256
experts, top-8 of softmax(router logits ~ N(0,1)), hidden 7168, expert
intermediate 256 (gate_up N=512 K=7168; down N=7168 K=256), INT4 weights with
group 128, fp16 scales and zero point 8, activations bf16 or fp8 e4m3 with
per-token scales -- for T in {1, 32, 512, 4096} tokens (every token at T = 512,
sampled tokens at T = 4096), plus small layers checked on every token.  The
unaligned path (hq_moe_gemm_by_slot: rows indexed by routed slot) is checked
the same way at decode-sized T.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_repack_amd as hq
import datagen
from oracle import gemm as og
from oracle import moe as om
from oracle import quant as oq
from oracle.formats import e4m3_value

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
E_FULL, H_FULL, I_FULL, TOPK = 256, 7168, 256, 8


def _log(msg):
    print(f"[gpu case] {msg}", flush=True)


# ------------------------------------------------------------------ align --

@pytest.mark.parametrize("T", [1, 32, 512, 4096])
def test_align_invariants(T):
    _log(f"moe align T={T}")
    r = datagen.moe_routing(T)
    ids = torch.from_numpy(r["topk_ids"]).to(DEV)
    sid, bexp, npad = hq.moe_align(ids, E_FULL, 16)
    torch.cuda.synchronize()
    om.check_align(r["topk_ids"], E_FULL, 16, sid.cpu().numpy(), bexp.cpu().numpy(), npad.cpu().numpy())


def test_align_out_of_range_ids():
    _log("moe align out-of-range ids")
    ids = np.array([[0, -1], [3, 4], [2, 0], [-1, 7], [1, 1], [9, 9]], dtype=np.int32)
    for bm in (16, 64):
        sid, bexp, npad = hq.moe_align(torch.from_numpy(ids).to(DEV), 4, bm)
        torch.cuda.synchronize()
        om.check_align(ids, 4, bm, sid.cpu().numpy(), bexp.cpu().numpy(), npad.cpu().numpy())


def test_align_extreme_ids():
    _log("moe align extreme ids")
    # any id outside [0, E) belongs to the trailing segment, including the
    # int32 extremes
    ids = np.array([[0, np.iinfo(np.int32).min], [3, np.iinfo(np.int32).max], [2, -1]] * 50, dtype=np.int32)
    for bm in (16, 64):
        sid, bexp, npad = hq.moe_align(torch.from_numpy(ids).to(DEV), 4, bm)
        torch.cuda.synchronize()
        om.check_align(ids, 4, bm, sid.cpu().numpy(), bexp.cpu().numpy(), npad.cpu().numpy())


def test_align_degenerate_cases():
    _log("moe align degenerate")
    # every slot on one expert; one expert only; block of 64
    ids = np.full((100, 4), 3, dtype=np.int32)
    sid, bexp, npad = hq.moe_align(torch.from_numpy(ids).to(DEV), 8, 16)
    torch.cuda.synchronize()
    om.check_align(ids, 8, 16, sid.cpu().numpy(), bexp.cpu().numpy(), npad.cpu().numpy())
    ids1 = np.zeros((7, 1), dtype=np.int32)
    sid, bexp, npad = hq.moe_align(torch.from_numpy(ids1).to(DEV), 1, 64)
    torch.cuda.synchronize()
    om.check_align(ids1, 1, 64, sid.cpu().numpy(), bexp.cpu().numpy(), npad.cpu().numpy())


# --------------------------------------------------------- layer pipeline --

def _quant(act, zp="fixed", scale="f16"):
    if act in ("bf16", "f16"):
        return hq.w4a16(act, scale=scale, zp=zp)
    return hq.w4a8_fp8(scale=scale, zp=zp)


def _out_fmt(act):
    return "f16" if act == "f16" else "bf16"


ACTS = ("bf16", "fp8", "f16")


class Layer:
    """Weights on the GPU (repacked for both activation types) + host copies.
    `tuning` (same for both GEMMs) forces a kernel / block size."""

    def __init__(self, E, H, I, key, tuning=None, max_t=4096, acts=ACTS, zp="fixed", scale="f16"):
        self.E, self.H, self.I = E, H, I
        wts = datagen.moe_weights(E, H, I, key=key, zp=zp)
        if scale == "bf16":  # the scales as bf16 values (rounded once; the oracle reads the same values)
            wts["s1"], wts["s2"] = wts["s1"].to(torch.bfloat16), wts["s2"].to(torch.bfloat16)
        self.w = wts
        # the oracle's zero points: fixed 8, or the per-group arrays
        self.z1, self.z2 = (wts["z1"], wts["z2"]) if zp == "u4" else (8, 8)
        self.dev = {}
        for act in acts:
            p1 = hq.MoePlan(2 * I, H, _quant(act, zp, scale), E, max_t,
                            "silu_mul_qfp8" if act == "fp8" else "silu_mul", tuning=tuning)
            p2 = hq.MoePlan(H, I, _quant(act, zp, scale), E, max_t, "topk_combine", tuning=tuning)
            z1 = torch.from_numpy(wts["z1"]).to(DEV) if zp == "u4" else None
            z2 = torch.from_numpy(wts["z2"]).to(DEV) if zp == "u4" else None
            w1, m1 = p1.repack(torch.from_numpy(wts["w1"]).to(DEV), wts["s1"].to(DEV), z1)
            w2, m2 = p2.repack(torch.from_numpy(wts["w2"]).to(DEV), wts["s2"].to(DEV), z2)
            self.dev[act] = (p1, p2, w1, m1, w2, m2)
        torch.cuda.synchronize()


def run_layer(layer, T, act, topk, key=(5,), sample=None, masked=0.0):
    """Run align -> gate_up -> down on the GPU; check every stage on sampled tokens.
    `masked`: fraction of slots whose expert id is replaced by an out-of-range
    one (-1 or E + 3); those slots must add nothing to y."""
    E, H, I = layer.E, layer.H, layer.I
    _log(f"moe layer E={E} H={H} I={I} T={T} topk={topk} act={act} block_m={layer.dev[act][0].block_m(T, topk)} "
         f"masked={masked}")
    r = datagen.moe_routing(T, E=E, topk=topk, key=key)
    if masked:
        rng = np.random.default_rng(99)
        ids = r["topk_ids"].copy()
        hit = rng.random(ids.shape) < masked
        ids[hit] = np.where(rng.random(ids.shape) < 0.5, -1, E + 3)[hit]
        r = dict(r, topk_ids=ids)
    x = datagen.moe_activations(T, H=H, act=act, key=key)
    p1, p2, w1, m1, w2, m2 = layer.dev[act]
    ids = torch.from_numpy(r["topk_ids"]).to(DEV)
    bm = p1.block_m(T, topk)
    assert p2.block_m(T, topk) == bm
    sid, bexp, npad = hq.moe_align(ids, E, bm)
    if act != "fp8":
        a = x["x"].to(DEV)
        act_out = p1.moe_gemm(a, T, topk, sid, bexp, npad, w1, m1)
        y = p2.moe_gemm(act_out, T, topk, sid, bexp, npad, w2, m2, topk_w=torch.from_numpy(r["topk_w"]).to(DEV))
    else:
        a = x["x_codes"].to(DEV)
        codes, scl = p1.moe_gemm(a, T, topk, sid, bexp, npad, w1, m1, a_scale=x["x_scale"].to(DEV))
        y = p2.moe_gemm(codes, T, topk, sid, bexp, npad, w2, m2, a_scale=scl,
                        topk_w=torch.from_numpy(r["topk_w"]).to(DEV))
    torch.cuda.synchronize()
    sid_h, bexp_h, npad_h = sid.cpu().numpy(), bexp.cpu().numpy(), int(npad.cpu().numpy()[0])
    om.check_align(r["topk_ids"], E, bm, sid_h, bexp_h, np.array([npad_h]))

    toks = np.arange(T) if sample is None or T <= sample else \
        np.sort(np.random.default_rng(T).choice(T, sample, replace=False))
    tokset = set(int(t) for t in toks)
    rows = [i for i in range(npad_h) if sid_h[i] < T * topk and int(sid_h[i]) // topk in tokset]
    rows = np.array(rows, dtype=np.int64)
    slot = sid_h[rows]
    flat = r["topk_ids"].reshape(-1)
    in_range = (flat[slot] >= 0) & (flat[slot] < E)
    assert np.array_equal(bexp_h[rows // bm], np.where(in_range, flat[slot], -1))
    rows, slot = rows[in_range], slot[in_range]  # out-of-range slots: no gate_up row, nothing in y
    row_tok = slot // topk
    row_exp = bexp_h[rows // bm]

    # gate_up: oracle on the GPU's stage input (the same x)
    if act != "fp8":
        xa = x["x"].double().numpy()[row_tok]
    else:
        xa = e4m3_value(x["x_codes"].numpy()[row_tok]) * x["x_scale"].numpy()[row_tok, None].astype(np.float64)
    gu = om.gate_up(xa, row_exp, layer.w["w1"], layer.w["s1"].double().numpy(), I, w1_zeros=layer.z1)
    if act != "fp8":
        act_gpu = act_out.double().cpu().numpy()[rows]
        ok, _, ratio = og.check(act_gpu, gu["act"], gu["tau_act"], _out_fmt(act))
        assert ok.all(), f"gate_up act: {(~ok).sum()} bad, max err/tau {ratio.max():.3g}"
        act_rows = act_gpu
    else:
        codes_h, scl_h = codes.cpu().numpy()[rows], scl.cpu().numpy()[rows]
        # the fp32 act rows the epilogue formed (the first max_padded * I * 4
        # bytes of the workspace) against the oracle's act
        mp = sid.numel()
        ws = p1.moe_workspace(T, topk, a.device)
        act32 = ws[: mp * I * 4].view(torch.float32).view(mp, I).cpu().numpy()[rows]
        err32 = np.abs(act32.astype(np.float64) - gu["act"])
        assert (err32 <= gu["tau_act"] + 2.0 ** -20 * np.abs(gu["act"])).all(), \
            f"gate_up fp32 act: {(err32 > gu['tau_act']).sum()} bad"
        # the requant follows the per-token quantiser's rule bit for bit on those rows
        qc, qs = oq.quantize_rows(act32, "fp8")
        assert np.array_equal(codes_h, qc), f"fp8 requant codes: {(codes_h != qc).sum()} differ from the rule"
        assert np.array_equal(scl_h, qs), "fp8 requant scales differ from the rule"
        # the scale against the oracle act's row maximum (a stale or inflated
        # maximum would miss this)
        s64 = np.abs(gu["act"]).max(1) / 448.0
        slack = (gu["tau_act"] + 2.0 ** -20 * np.abs(gu["act"])).max(1) / 448.0 + 2.0 ** -22 * s64
        assert (np.abs(scl_h - s64) <= slack).all(), "fp8 requant scale off the oracle's row maximum"
        dq = e4m3_value(codes_h) * scl_h[:, None].astype(np.float64)
        bound = om.fp8_rows_bound(dq, scl_h, gu["act"], gu["tau_act"])
        err = np.abs(dq - gu["act"])
        assert (err <= bound).all(), f"fp8 requant: {(err > bound).sum()} bad"
        act_rows = dq
    # down + combine: oracle on the GPU's act rows, for the sampled tokens
    # the aligned path stores each weighted slot row in bf16 before the combine
    dc = om.down_combine(act_rows, row_tok, r["topk_w"].reshape(-1)[slot], row_exp, layer.w["w2"],
                         layer.w["s2"].double().numpy(), T, rows_fmt="bf16", topk=topk, w2_zeros=layer.z2)
    y_gpu = y.double().cpu().numpy()[toks]
    ok, _, ratio = og.check(y_gpu, dc["y64"][toks], dc["tau_y"][toks], _out_fmt(act))
    assert ok.all(), f"down+combine: {(~ok).sum()} bad, max err/tau {ratio.max():.3g}"
    return ratio.max()


def run_layer_by_slot(layer, T, act, topk, key=(5,), sample=None, masked=0.0, ws=None):
    """gate_up -> down through hq_moe_gemm_by_slot (rows indexed by routed slot,
    no alignment); every stage checked against the oracle on the GPU's own
    input to it, for all tokens or a sample.  Slots with an out-of-range
    expert id must give a zero gate_up row and add nothing to y."""
    E, H, I = layer.E, layer.H, layer.I
    _log(f"moe by-slot E={E} H={H} I={I} T={T} topk={topk} act={act} masked={masked}")
    r = datagen.moe_routing(T, E=E, topk=topk, key=key)
    if masked:
        rng = np.random.default_rng(98)
        ids = r["topk_ids"].copy()
        hit = rng.random(ids.shape) < masked
        ids[hit] = np.where(rng.random(ids.shape) < 0.5, -1, E + 3)[hit]
        r = dict(r, topk_ids=ids)
    x = datagen.moe_activations(T, H=H, act=act, key=key)
    p1, p2, w1, m1, w2, m2 = layer.dev[act]
    ids = torch.from_numpy(r["topk_ids"]).to(DEV)
    tw = torch.from_numpy(r["topk_w"]).to(DEV)
    S = T * topk
    if act != "fp8":
        act_out = p1.moe_gemm_by_slot(x["x"].to(DEV), T, topk, ids, w1, m1)
        y = p2.moe_gemm_by_slot(act_out, T, topk, ids, w2, m2, topk_w=tw)
    else:
        if ws is None:
            ws = p1.moe_workspace(T, topk, DEV)
        codes, scl = p1.moe_gemm_by_slot(x["x_codes"].to(DEV), T, topk, ids, w1, m1, a_scale=x["x_scale"].to(DEV),
                                         ws=ws)
        y = p2.moe_gemm_by_slot(codes, T, topk, ids, w2, m2, a_scale=scl, topk_w=tw)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T, H)

    toks = np.arange(T) if sample is None or T <= sample else \
        np.sort(np.random.default_rng(T).choice(T, sample, replace=False))
    slots = (toks[:, None] * topk + np.arange(topk)[None, :]).reshape(-1)
    flat = r["topk_ids"].reshape(-1)
    valid = (flat[slots] >= 0) & (flat[slots] < E)
    vs, bad = slots[valid], slots[~valid]
    row_tok, row_exp = vs // topk, flat[vs]
    if act != "fp8":
        xa = x["x"].double().numpy()[row_tok]
    else:
        xa = e4m3_value(x["x_codes"].numpy()[row_tok]) * x["x_scale"].numpy()[row_tok, None].astype(np.float64)
    gu = om.gate_up(xa, row_exp, layer.w["w1"], layer.w["s1"].double().numpy(), I, w1_zeros=layer.z1)
    if act != "fp8":
        assert tuple(act_out.shape) == (S, I)
        out_h = act_out.double().cpu().numpy()
        act_rows = out_h[vs]
        ok, _, ratio = og.check(act_rows, gu["act"], gu["tau_act"], _out_fmt(act))
        assert ok.all(), f"gate_up act: {(~ok).sum()} bad, max err/tau {ratio.max():.3g}"
        assert (out_h[bad] == 0).all(), "rows of out-of-range slots must be zero"
    else:
        assert tuple(codes.shape) == (S, I) and tuple(scl.shape) == (S,)
        codes_a, scl_a = codes.cpu().numpy(), scl.cpu().numpy()
        act32_a = ws[: S * I * 4].view(torch.float32).view(S, I).cpu().numpy()
        act32, codes_h, scl_h = act32_a[vs], codes_a[vs], scl_a[vs]
        err32 = np.abs(act32.astype(np.float64) - gu["act"])
        assert (err32 <= gu["tau_act"] + 2.0 ** -20 * np.abs(gu["act"])).all(), \
            f"gate_up fp32 act: {(err32 > gu['tau_act']).sum()} bad"
        qc, qs = oq.quantize_rows(act32, "fp8")
        assert np.array_equal(codes_h, qc), f"fp8 requant codes: {(codes_h != qc).sum()} differ from the rule"
        assert np.array_equal(scl_h, qs), "fp8 requant scales differ from the rule"
        assert (codes_a[bad] == 0).all() and (scl_a[bad] == 1.0).all(), "out-of-range slots: zero codes, scale 1"
        dq = e4m3_value(codes_h) * scl_h[:, None].astype(np.float64)
        bound = om.fp8_rows_bound(dq, scl_h, gu["act"], gu["tau_act"])
        assert (np.abs(dq - gu["act"]) <= bound).all(), "fp8 requant off the oracle's act"
        act_rows = dq
    dc = om.down_combine(act_rows, row_tok, r["topk_w"].reshape(-1)[vs], row_exp, layer.w["w2"],
                         layer.w["s2"].double().numpy(), T, w2_zeros=layer.z2)
    y_gpu = y.double().cpu().numpy()[toks]
    ok, _, ratio = og.check(y_gpu, dc["y64"][toks], dc["tau_y"][toks], _out_fmt(act))
    assert ok.all(), f"down+combine by slot: {(~ok).sum()} bad, max err/tau {ratio.max():.3g}"
    return ratio.max()


@pytest.fixture(scope="module")
def small_layer():
    return Layer(8, 512, 128, key=(7,))


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("T,topk", [(1, 2), (37, 2), (200, 3), (5, 8)])
def test_small_layer_all_tokens(small_layer, T, topk, act):
    run_layer(small_layer, T, act, topk, key=(11,))


@pytest.fixture(scope="module")
def small_layer_zp():
    # per-group uint4 zero points (6..9) on every expert
    return Layer(8, 512, 128, key=(9,), zp="u4")


@pytest.fixture(scope="module")
def small_layer_bf16_scales():
    return Layer(8, 512, 128, key=(10,), scale="bf16", zp="u4")


@pytest.mark.parametrize("act", ACTS)
def test_small_layer_bf16_scales_aligned_and_by_slot(small_layer_bf16_scales, act):
    run_layer(small_layer_bf16_scales, 40, act, 2, key=(97,))
    run_layer_by_slot(small_layer_bf16_scales, 3, act, 8, key=(97,))


@pytest.fixture(scope="module")
def small_layer_zp_tiled():
    return Layer(8, 512, 128, key=(9,), zp="u4", tuning=dict(kernel=2, tile_m=64, tile_n=256))


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("T,topk", [(1, 2), (37, 2), (5, 8)])
def test_small_layer_group_zero_points(small_layer_zp, T, topk, act):
    run_layer(small_layer_zp, T, act, topk, key=(79,))


@pytest.mark.parametrize("act", ACTS)
def test_small_layer_group_zero_points_tiled(small_layer_zp_tiled, act):
    run_layer(small_layer_zp_tiled, 200, act, 3, key=(83,))


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("T,topk", [(1, 8), (6, 4)])
def test_small_layer_group_zero_points_by_slot(small_layer_zp, T, topk, act):
    run_layer_by_slot(small_layer_zp, T, act, topk, key=(89,), masked=0.2 if T > 1 else 0.0)


@pytest.fixture(scope="module")
def small_layer_32():
    return Layer(8, 512, 128, key=(7,), tuning=dict(kernel=1, tile_m=32))


@pytest.mark.parametrize("act", ["bf16", "fp8"])
@pytest.mark.parametrize("T,topk", [(1, 2), (37, 2), (150, 3)])
def test_small_layer_32_row_blocks(small_layer_32, T, topk, act):
    # the weight-streaming kernel with two 16-row blocks per workgroup
    run_layer(small_layer_32, T, act, topk, key=(23,))


# the MFMA-tiled grouped kernel on every token: 64- and 128-row blocks, 128-
# and 256-column tiles (gate_up n = 256: one or two paired tiles; down K = 128:
# a single k group), mostly-empty blocks at small T
TILED = [dict(kernel=2, tile_m=64, tile_n=128), dict(kernel=2, tile_m=128, tile_n=128),
         dict(kernel=2, tile_m=64, tile_n=256)]


@pytest.fixture(scope="module", params=range(len(TILED)), ids=["bm64_bn128", "bm128_bn128", "bm64_bn256"])
def small_layer_tiled(request):
    return Layer(8, 512, 128, key=(7,), tuning=TILED[request.param])


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("T,topk", [(3, 2), (200, 3), (700, 2)])
def test_small_layer_tiled(small_layer_tiled, T, topk, act):
    run_layer(small_layer_tiled, T, act, topk, key=(17,))


@pytest.mark.parametrize("act", ["bf16", "fp8"])
@pytest.mark.parametrize("T,topk,tiled", [(40, 3, False), (300, 2, True)])
def test_small_layer_masked_experts(small_layer, small_layer_tiled, T, topk, tiled, act):
    # slots routed to -1 or past the last expert: dropped from the combine
    run_layer(small_layer_tiled if tiled else small_layer, T, act, topk, key=(19,), masked=0.15)


def test_small_layer_repeat_calls_reuse_workspace(small_layer):
    # calls in a row on the same plans and workspace all pass: nothing a call
    # leaves in the workspace is read by the next one
    for act in ("fp8", "bf16", "fp8"):
        run_layer(small_layer, 64, act, 2, key=(13,))


@pytest.mark.parametrize("tiled", [False, True])
def test_fp8_requant_with_fewer_tokens_than_the_call_before(small_layer, small_layer_tiled, tiled):
    # a large call fills the workspace, then smaller ones (other t, topk, block
    # size) reuse it: their scales must come from their own rows
    lay = small_layer_tiled if tiled else small_layer
    for T, topk in ((400, 3), (5, 8), (1, 2), (64, 2)):
        run_layer(lay, T, "fp8", topk, key=(29,))


@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_small_layer_many_slots_column_windows(act):
    # 524288 routed slots of 2048 columns: the down GEMM and the combine run
    # in two column windows (the weighted bf16 slot rows of one window stay
    # within 1 GiB of workspace), checked on sampled tokens
    lay = Layer(8, 2048, 128, key=(31,), max_t=65536, tuning=dict(tile_m=64))
    run_layer(lay, 65536, act, 8, key=(37,), sample=24)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("T,topk", [(1, 2), (1, 8), (3, 8), (37, 2), (200, 3), (1, 1), (9, 1)])
def test_small_layer_by_slot(small_layer, T, topk, act):
    run_layer_by_slot(small_layer, T, act, topk, key=(41,))


@pytest.mark.parametrize("act", ["bf16", "fp8"])
@pytest.mark.parametrize("T,topk", [(1, 8), (40, 3)])
def test_small_layer_by_slot_masked_experts(small_layer, T, topk, act):
    run_layer_by_slot(small_layer, T, act, topk, key=(43,), masked=0.3)


@pytest.mark.parametrize("tun", [dict(tile_n=16, waves=1), dict(tile_n=32, waves=16), dict(tile_n=64, waves=5)],
                         ids=["n16w1", "n32w16", "n64w5"])
@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_small_layer_by_slot_tunings(tun, act):
    # every column-block width and wave count the by-slot kernels take
    run_layer_by_slot(Layer(8, 512, 128, key=(7,), tuning=tun), 6, act, 4, key=(47,))


@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_small_layer_plain_epilogue_aligned_and_by_slot(small_layer, act):
    # the grouped GEMM without an activation (epilogue "none"): rows x_tok . W1_e^T of
    # every slot, by aligned position and by slot; a masked slot gives no aligned row
    # and a zero row by slot
    lay = small_layer
    E, H, I, T, topk = lay.E, lay.H, lay.I, 9, 3
    _log(f"moe plain epilogue T={T} topk={topk} act={act}")
    r = datagen.moe_routing(T, E=E, topk=topk, key=(61,))
    ids_h = r["topk_ids"].copy()
    ids_h[0, 1] = -1
    x = datagen.moe_activations(T, H=H, act=act, key=(61,))
    w1, m1 = lay.dev[act][2], lay.dev[act][3]
    p = hq.MoePlan(2 * I, H, _quant(act), E, 4096, "none")
    ids = torch.from_numpy(ids_h).to(DEV)
    a = (x["x"] if act != "fp8" else x["x_codes"]).to(DEV)
    xs = None if act != "fp8" else x["x_scale"].to(DEV)
    sid, bex, npad = hq.moe_align(ids, E, p.block_m(T, topk))
    out_al = p.moe_gemm(a, T, topk, sid, bex, npad, w1, m1, a_scale=xs)
    out_sl = p.moe_gemm_by_slot(a, T, topk, ids, w1, m1, a_scale=xs)
    torch.cuda.synchronize()
    if act != "fp8":
        xt = x["x"].double().numpy()
    else:
        xt = e4m3_value(x["x_codes"].numpy()) * x["x_scale"].numpy()[:, None].astype(np.float64)
    flat = ids_h.reshape(-1)
    slots = np.nonzero((flat >= 0) & (flat < E))[0]
    o, tau = om.grouped_gemm(xt[slots // topk], flat[slots], lay.w["w1"], lay.w["s1"].double().numpy(), lay.z1)
    sl = out_sl.double().cpu().numpy()
    assert sl.shape == (T * topk, 2 * I)
    ok, _, ratio = og.check(sl[slots], o, tau, _out_fmt(act))
    assert ok.all(), f"by slot: {(~ok).sum()} bad, max err/tau {ratio.max():.3g}"
    assert (sl[~np.isin(np.arange(T * topk), slots)] == 0).all()
    sid_h = sid.cpu().numpy()
    pos = {int(v): i for i, v in enumerate(sid_h[: int(npad.cpu()[0])]) if v < T * topk}
    al = out_al.double().cpu().numpy()[[pos[int(v)] for v in slots]]
    ok, _, ratio = og.check(al, o, tau, _out_fmt(act))
    assert ok.all(), f"aligned: {(~ok).sum()} bad, max err/tau {ratio.max():.3g}"


@pytest.mark.parametrize("act", ["bf16", "fp8"])
@pytest.mark.parametrize("T,topk", [(2, 8), (14, 8), (60, 3)])
def test_moe_layer_helper_matches_its_path(small_layer, T, topk, act):
    # hq.moe_layer picks the by-slot path for few routed slots, the aligned one
    # otherwise, and returns what the explicit calls of that path return
    lay = small_layer
    _log(f"moe_layer helper T={T} topk={topk} act={act}")
    r = datagen.moe_routing(T, E=lay.E, topk=topk, key=(67,))
    x = datagen.moe_activations(T, H=lay.H, act=act, key=(67,))
    p1, p2, w1, m1, w2, m2 = lay.dev[act]
    ids = torch.from_numpy(r["topk_ids"]).to(DEV)
    tw = torch.from_numpy(r["topk_w"]).to(DEV)
    a = (x["x"] if act != "fp8" else x["x_codes"]).to(DEV)
    xs = None if act != "fp8" else x["x_scale"].to(DEV)
    y = hq.moe_layer(p1, p2, a, ids, tw, w1, m1, w2, m2, x_scale=xs)
    by_slot = hq.moe_uses_by_slot(T, topk, act == "fp8")
    assert by_slot == (T * topk <= (96 if act == "fp8" else 128))
    if by_slot:
        res = p1.moe_gemm_by_slot(a, T, topk, ids, w1, m1, a_scale=xs)
        act_out, scl = res if act == "fp8" else (res, None)
        ref = p2.moe_gemm_by_slot(act_out, T, topk, ids, w2, m2, a_scale=scl, topk_w=tw)
    else:
        sid, bex, npad = hq.moe_align(ids, lay.E, p1.block_m(T, topk))
        res = p1.moe_gemm(a, T, topk, sid, bex, npad, w1, m1, a_scale=xs)
        act_out, scl = res if act == "fp8" else (res, None)
        ref = p2.moe_gemm(act_out, T, topk, sid, bex, npad, w2, m2, a_scale=scl, topk_w=tw)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


def test_by_slot_fp8_workspace_reuse(small_layer):
    # one workspace across calls of falling size: each call's scales come from its own rows
    ws = small_layer.dev["fp8"][0].moe_workspace(64, 8, DEV)
    for T, topk in ((64, 8), (5, 3), (1, 8), (2, 2)):
        run_layer_by_slot(small_layer, T, "fp8", topk, key=(53,), ws=ws)


@pytest.fixture(scope="module")
def full_layer():
    _log("generating the 256-expert layer")
    return Layer(E_FULL, H_FULL, I_FULL, key=(5,))


@pytest.mark.parametrize("act", ["bf16", "fp8"])
@pytest.mark.parametrize("T", [1, 32, 512, 4096])
def test_full_layer(full_layer, T, act):
    run_layer(full_layer, T, act, TOPK, sample=12)


@pytest.mark.parametrize("act", ["bf16", "fp8"])
@pytest.mark.parametrize("T", [1, 2, 4, 8, 32])
def test_full_layer_by_slot(full_layer, T, act):
    # decode-sized batches through the unaligned path, every token
    run_layer_by_slot(full_layer, T, act, TOPK)


@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_full_layer_by_slot_masked(full_layer, act):
    run_layer_by_slot(full_layer, 4, act, TOPK, key=(59,), masked=0.25)


@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_full_layer_t512_every_token(full_layer, act):
    # all 512 tokens (4096 routed slots, every expert hit), stage by stage
    run_layer(full_layer, 512, act, TOPK, sample=None)


@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_full_layer_tiled_128_rows(full_layer, act):
    # T = 4096 again with the other tiled block size (and 256-column tiles)
    tl = Layer.__new__(Layer)
    tl.E, tl.H, tl.I, tl.w = full_layer.E, full_layer.H, full_layer.I, full_layer.w
    tl.z1, tl.z2 = full_layer.z1, full_layer.z2
    tl.dev = {}
    for a in ("bf16", "fp8"):
        _, _, w1, m1, w2, m2 = full_layer.dev[a]
        tun = dict(kernel=2, tile_m=128, tile_n=256)
        p1 = hq.MoePlan(2 * tl.I, tl.H, _quant(a), tl.E, 4096, "silu_mul_qfp8" if a == "fp8" else "silu_mul",
                        tuning=tun)
        p2 = hq.MoePlan(tl.H, tl.I, _quant(a), tl.E, 4096, "topk_combine", tuning=tun)
        tl.dev[a] = (p1, p2, w1, m1, w2, m2)
    run_layer(tl, 4096, act, TOPK, sample=12)
