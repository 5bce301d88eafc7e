"""HIP-graph capture of the library's calls, the way a decode loop runs them:
decode GEMMs (with a K split: GEMM + split-K reduce; with staged activation
rows), the aligned MoE layer
(align, gate_up with the fp8 requant, down, combine) and the by-slot MoE layer.
Each sequence is captured once and replayed several times; before every replay
new inputs are copied into the captured input buffers, the program does eager
work of its own and synchronises, and every replay's outputs must equal the
eager calls on the same inputs bit for bit (the kernels are deterministic).
None of these paths records a memset into the graph."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_repack_amd as hq
import datagen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 4


def _log(msg):
    print(f"[gpu case] {msg}", flush=True)


def _replay_and_check(capture_calls, set_inputs, outputs, eager_calls, eager_outputs):
    """capture_calls() launches the sequence on the captured buffers; set_inputs(i)
    writes input set i into them; eager_calls() runs the same sequence into
    eager_outputs from the same inputs."""
    set_inputs(0)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        capture_calls()                    # warm-up outside the capture (plans, attributes)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture_calls()
    for i in range(REPLAYS):
        set_inputs(i + 1)
        scratch = torch.randn(1 << 20, device=DEV)     # eager work of the program's own between replays
        scratch.mul_(2.0).add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        eager_calls()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, eager_outputs)):
            assert torch.equal(a, b), f"replay {i}: output {k} differs from the eager calls"
        assert all(torch.isfinite(o.float()).all() for o in got if o.dtype != torch.uint8)
    del g


@pytest.mark.parametrize("M", [16, 1])
def test_graph_decode_gemm(M):
    # M = 16 takes the K split and its reduce; M = 1 the activation rows staged
    # in LDS (a slab of 28 KiB behind the reduction buffer)
    N, K = 4096, 14336
    _log(f"graph decode gemm M={M} N={N} K={K}")
    d = datagen.dense_w4a16(M, N, K, act="bf16", zp="u4", key=(71,))
    p = hq.Plan(N, K, hq.w4a16(act="bf16", zp="u4"), max_m=M)
    assert ("split_k=1 " not in p.describe(M) + " ") == (M == 16)
    w, meta = p.repack(torch.from_numpy(d["codes"]).to(DEV), d["scales"].to(DEV), torch.from_numpy(d["zeros"]).to(DEV))
    a = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    out, ref = (torch.empty((M, N), dtype=torch.bfloat16, device=DEV) for _ in range(2))
    ws = p.workspace(M, DEV)
    gen = torch.Generator(device="cpu").manual_seed(5)
    inputs = [torch.randn((M, K), generator=gen).to(torch.bfloat16) for _ in range(REPLAYS + 1)]
    cur = {}

    def set_inputs(i):
        a.copy_(inputs[i].to(DEV))
        cur["i"] = i

    _replay_and_check(lambda: p.gemm(a, w, meta, out=out, ws=ws), set_inputs, [out],
                      lambda: p.gemm(inputs[cur["i"]].to(DEV), w, meta, out=ref, ws=ws), [ref])


class _Moe:
    def __init__(self, act, E=8, H=512, I=128):
        self.E, self.H, self.I, self.act = E, H, I, act
        q = hq.w4a16("bf16", scale="f16") if act == "bf16" else hq.w4a8_fp8(scale="f16")
        wts = datagen.moe_weights(E, H, I, key=(73,))
        self.p1 = hq.MoePlan(2 * I, H, q, E, 512, "silu_mul" if act == "bf16" else "silu_mul_qfp8")
        self.p2 = hq.MoePlan(H, I, q, E, 512, "topk_combine")
        self.w1, self.m1 = self.p1.repack(torch.from_numpy(wts["w1"]).to(DEV), wts["s1"].to(DEV))
        self.w2, self.m2 = self.p2.repack(torch.from_numpy(wts["w2"]).to(DEV), wts["s2"].to(DEV))

    def inputs(self, T, topk, n):
        sets = []
        for j in range(n):
            r = datagen.moe_routing(T, E=self.E, topk=topk, key=(75, j))
            x = datagen.moe_activations(T, H=self.H, act=self.act, key=(75, j))
            xa = x["x"] if self.act == "bf16" else x["x_codes"]
            xs = None if self.act == "bf16" else x["x_scale"]
            sets.append((torch.from_numpy(r["topk_ids"]), torch.from_numpy(r["topk_w"]), xa, xs))
        return sets


@pytest.mark.parametrize("act", ["bf16", "fp8"])
@pytest.mark.parametrize("T,topk", [(24, 2), (400, 2)], ids=["skinny", "tiled"])
def test_graph_moe_layer_aligned(act, T, topk):
    # 24 tokens take the weight-streaming kernels, 400 (100 slots per expert)
    # the persistent tiled gate_up and the small-K down
    _log(f"graph moe aligned T={T} topk={topk} act={act}")
    m = _Moe(act)
    assert ("grouped-tiled" in m.p1.describe(T, topk)) == (T == 400)
    E, I = m.E, m.I
    bm = m.p1.block_m(T, topk)
    mp = hq.moe_max_padded(T, topk, E, bm)
    sets = m.inputs(T, topk, REPLAYS + 1)
    ids = torch.empty((T, topk), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, topk), dtype=torch.float32, device=DEV)
    xa = torch.empty(sets[0][2].shape, dtype=sets[0][2].dtype, device=DEV)
    xs = None if act == "bf16" else torch.empty(T, dtype=torch.float32, device=DEV)
    ws1, ws2 = m.p1.moe_workspace(T, topk, DEV), m.p2.moe_workspace(T, topk, DEV)
    L = hq.lib()

    def buffers():
        return dict(sid=torch.empty(mp, dtype=torch.int32, device=DEV),
                    bex=torch.empty(max(mp // bm, 1), dtype=torch.int32, device=DEV),
                    npad=torch.empty(1, dtype=torch.int32, device=DEV),
                    inter=torch.empty((mp, I), dtype=torch.bfloat16 if act == "bf16" else torch.uint8, device=DEV),
                    iscale=None if act == "bf16" else torch.empty(mp, dtype=torch.float32, device=DEV),
                    y=torch.empty((T, m.H), dtype=torch.bfloat16, device=DEV))

    cap, eag = buffers(), buffers()

    def layer(b):
        hq._check(L.hq_moe_align(T, topk, E, bm, hq._ptr(ids), hq._ptr(b["sid"]), hq._ptr(b["bex"]),
                                 hq._ptr(b["npad"]), hq._stream_ptr(ids.device)))
        m.p1.moe_gemm(xa, T, topk, b["sid"], b["bex"], b["npad"], m.w1, m.m1, a_scale=xs, out=b["inter"],
                      out_scale=b["iscale"], ws=ws1)
        m.p2.moe_gemm(b["inter"], T, topk, b["sid"], b["bex"], b["npad"], m.w2, m.m2, a_scale=b["iscale"],
                      topk_w=tw, out=b["y"], ws=ws2)

    def set_inputs(i):
        ids.copy_(sets[i][0].to(DEV))
        tw.copy_(sets[i][1].to(DEV))
        xa.copy_(sets[i][2].to(DEV))
        if xs is not None:
            xs.copy_(sets[i][3].to(DEV))

    # the aligned slot order inside a segment is unspecified, so the replay is
    # compared on y (and on the used length), which do not depend on it
    _replay_and_check(lambda: layer(cap), set_inputs, [cap["y"], cap["npad"]], lambda: layer(eag),
                      [eag["y"], eag["npad"]])


@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_graph_moe_layer_by_slot(act):
    T, topk = 3, 8
    _log(f"graph moe by slot T={T} topk={topk} act={act}")
    m = _Moe(act)
    S = T * topk
    sets = m.inputs(T, topk, REPLAYS + 1)
    ids = torch.empty((T, topk), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, topk), dtype=torch.float32, device=DEV)
    xa = torch.empty(sets[0][2].shape, dtype=sets[0][2].dtype, device=DEV)
    xs = None if act == "bf16" else torch.empty(T, dtype=torch.float32, device=DEV)
    ws1 = m.p1.moe_workspace(T, topk, DEV) if act == "fp8" else None

    def buffers():
        return dict(inter=torch.empty((S, m.I), dtype=torch.bfloat16 if act == "bf16" else torch.uint8, device=DEV),
                    iscale=None if act == "bf16" else torch.empty(S, dtype=torch.float32, device=DEV),
                    y=torch.empty((T, m.H), dtype=torch.bfloat16, device=DEV))

    cap, eag = buffers(), buffers()

    def layer(b):
        m.p1.moe_gemm_by_slot(xa, T, topk, ids, m.w1, m.m1, a_scale=xs, out=b["inter"], out_scale=b["iscale"],
                              ws=ws1)
        m.p2.moe_gemm_by_slot(b["inter"], T, topk, ids, m.w2, m.m2, a_scale=b["iscale"], topk_w=tw, out=b["y"])

    def set_inputs(i):
        ids.copy_(sets[i][0].to(DEV))
        tw.copy_(sets[i][1].to(DEV))
        xa.copy_(sets[i][2].to(DEV))
        if xs is not None:
            xs.copy_(sets[i][3].to(DEV))

    outs = ["inter", "y"] + ([] if act == "bf16" else ["iscale"])
    _replay_and_check(lambda: layer(cap), set_inputs, [cap[k] for k in outs], lambda: layer(eag),
                      [eag[k] for k in outs])
