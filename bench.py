#!/usr/bin/env python3
"""Benchmark of the dense W4A16 decode sweep on one MI355X.

Workload (one step): the twelve GEMMs of the decode sweep, M in {1, 4, 16, 64}
x (N, K) in {(4096, 4096), (14336, 4096), (4096, 14336)}, bf16 activations,
uint4 weights with group 128, bf16 group scales and uint4 zero points, bf16
output.  Inputs are seeded synthetic data (A ~ N(0,1), codes uniform 0..15,
scales uniform [0.005, 0.02], zeros uniform 6..9), resident in HBM before the
timed region.  Every launch reads its own copy of the weights from a rotating
pool (> 1 GB, four times the 256 MB last-level cache), so weights come from
HBM, not from a cache.

Timings
  * ms_per_step: K steps replayed as HIP graphs (one graph per pool rotation),
    bracketed by synchronisations, timed with events on the launch stream.
    `value` = algorithmic bytes of the sweep / ms_per_step (GB/s).
  * roofline: the same K steps launched eagerly, each hq_gemm call bracketed
    by HIP events recorded at the start of its first dispatch and the end of
    its last (hq_time_next_launch; a call is one GEMM kernel, plus the
    split-K reduce where K is split); achieved = algorithmic bytes per call /
    mean call duration.  traffic: HBM bytes per call from the committed
    FETCH_SIZE / WRITE_SIZE counter summary, used only while the kernel
    sources it was taken on are unchanged (source hash), else null.
  * cpu_baseline: the CPU oracle (oracle/, float64 dequantise + GEMM) on a
    bounded sample of the same points, on this host's cores.

Algorithmic bytes per GEMM: N*K/2 (codes) + 2*N*K/128 (bf16 scales) +
N*K/256 (4-bit zeros) + 2*M*K (A) + 2*M*N (C).  Flops: 2*M*N*K.

`--workload quant` measures the per-token activation quantiser instead (the
step before the W4A8 GEMMs): x bf16 [M, 7168] for M in {1, 16, 128, 1024},
fp8 and int8 codes, inputs rotated over 16 copies; algorithmic bytes per
launch 2*M*K (x) + M*K (codes) + 4*M (scales).  The default run is the decode
sweep.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

SWEEP_M = (1, 4, 16, 64)
SWEEP_NK = ((4096, 4096), (14336, 4096), (4096, 14336))
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "quantized GEMM TFLOPS and effective HBM GB/s (% of roofline) vs M"
WORKLOAD = ("dense W4A16 decode sweep: M in {1,4,16,64} x (N,K) in {(4096,4096),(14336,4096),(4096,14336)}, "
            "bf16 activations, uint4 weights (group 128, bf16 scales, uint4 zero points), bf16 output")


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qgemm_decode_sweep_traffic.json")


def kernel_source_hash():
    """sha256 over the library's kernel and host sources (sorted by name)."""
    import hashlib

    csrc = os.path.join(ROOT, "bit_quantized_gemm_repack_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per call from the counter summary, if taken on these sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_call")


def algo_bytes(M, N, K):
    return N * K // 2 + 2 * N * (K // 128) + N * (K // 128) // 2 + 2 * M * K + 2 * M * N


def algo_flops(M, N, K):
    return 2 * M * N * K


class Hip:
    """hipEvent helpers from the HIP runtime torch already loaded."""

    def __init__(self):
        torch.cuda.init()
        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.L = ctypes.CDLL(path)
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.L.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def make_points(dev, rotations):
    import bit_quantized_gemm_repack_amd as hq
    import datagen

    shapes = {}
    for (N, K) in SWEEP_NK:
        d = datagen.dense_w4a16(max(SWEEP_M), N, K, act="bf16", zp="u4", key=(2,))
        plan_any = hq.Plan(N, K, hq.w4a16(act="bf16", zp="u4"), max_m=max(SWEEP_M))
        w, meta = plan_any.repack(torch.from_numpy(d["codes"]).to(dev), d["scales"].to(dev),
                                  torch.from_numpy(d["zeros"]).to(dev))
        shapes[(N, K)] = dict(data=d, w=w, meta=meta)
    points = []
    # interleave shapes so that consecutive launches touch different weights
    for M in SWEEP_M:
        for (N, K) in SWEEP_NK:
            s = shapes[(N, K)]
            plan = hq.Plan(N, K, hq.w4a16(act="bf16", zp="u4"), max_m=M)
            a = s["data"]["a"][:M].contiguous().to(dev)
            copies = [(s["w"].clone(), s["meta"].clone()) for _ in range(rotations)]
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = plan.workspace(M, dev)
            points.append(dict(M=M, N=N, K=K, plan=plan, a=a, copies=copies, out=out, ws=ws,
                               bytes=algo_bytes(M, N, K), flops=algo_flops(M, N, K)))
    torch.cuda.synchronize()
    return points, shapes


def run_step(points, r):
    for p in points:
        w, meta = p["copies"][r]
        p["plan"].gemm(p["a"], w, meta, out=p["out"], ws=p["ws"])


def check_point(points, shapes):
    """Spot check of one point against the CPU oracle (sampled rows)."""
    from oracle import gemm as og

    p = next(q for q in points if q["M"] == 16 and q["N"] == 4096 and q["K"] == 4096)
    d = shapes[(4096, 4096)]["data"]
    ref = og.gemm_w4a16(d["a"][:16].double().numpy(), d["codes"], d["scales"].double().numpy(), d["zeros"],
                        out_fmt="bf16")
    ok, _, ratio = og.check(p["out"].double().cpu().numpy(), ref["c64"], ref["tau"], "bf16")
    if not ok.all():
        raise SystemExit(f"bench: output check failed ({int((~ok).sum())} outputs, max err/tau {ratio.max():.3g})")
    return float(ratio.max())


def cpu_baseline(budget_s: float):
    """Time the CPU oracle on points of the sweep until ~budget_s seconds."""
    import datagen
    from oracle import gemm as og

    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        blas_threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count() or 1
    done_bytes, secs, names = 0, 0.0, []
    order = [(M, N, K) for M in SWEEP_M for (N, K) in SWEEP_NK]
    for i in range(10 * len(order)):
        M, N, K = order[i % len(order)]
        d = datagen.dense_w4a16(M, N, K, act="bf16", zp="u4", key=(2,))
        a = d["a"].double().numpy()
        s = d["scales"].double().numpy()
        t0 = time.perf_counter()
        og.gemm_w4a16(a, d["codes"], s, d["zeros"], out_fmt="bf16")
        dt = time.perf_counter() - t0
        secs += dt
        done_bytes += algo_bytes(M, N, K)
        if f"M={M} N={N} K={K}" not in names:
            names.append(f"M={M} N={N} K={K}")
        runs = i + 1
        if secs >= budget_s:
            break
    return {"value": done_bytes / secs / 1e9, "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{runs} oracle runs over {len(names)} points of the sweep ({'; '.join(names)}), unpack + float64 dequantise + "
                      f"float64 GEMM incl. tolerance terms, {secs:.1f} s total; cores = BLAS threads "
                      f"(the dequantise step is single-threaded numpy)"}


QUANT_M = (1, 16, 128, 1024)
QUANT_K = 7168
QUANT_METRIC = "per-token activation quantiser effective HBM GB/s vs M"
QUANT_WORKLOAD = ("per-token activation quantiser (the W4A8 GEMMs' input step): x bf16 [M, 7168], "
                  "M in {1,16,128,1024}, fp8 e4m3 and int8 codes + fp32 row scales")


def quant_bytes(M, K):
    return 2 * M * K + M * K + 4 * M


def run_quant(args):
    """The quantiser workload: one step = 8 launches (each M, fp8 and int8)."""
    import bit_quantized_gemm_repack_amd as hq

    dev = torch.device("cuda:0")
    hip = Hip()
    L = hq.lib()
    # enough input copies that a step's rotation does not fit the 256 MB last-level cache
    R = max(args.rotations, 16)
    pts = []
    for M in QUANT_M:
        g = torch.Generator().manual_seed(M)
        x = torch.randn((M, QUANT_K), generator=g).to(torch.bfloat16)
        xs = [x.to(dev) for _ in range(R)]
        for out in ("fp8", "int8"):
            codes = torch.empty((M, QUANT_K), dtype=torch.uint8 if out == "fp8" else torch.int8, device=dev)
            scales = torch.empty(M, dtype=torch.float32, device=dev)
            pts.append(dict(M=M, out=out, xs=xs, codes=codes, scales=scales, bytes=quant_bytes(M, QUANT_K)))
    step_bytes = sum(p["bytes"] for p in pts)

    def step(r):
        for p in pts:
            hq.quantize_per_token(p["xs"][r], p["out"], codes=p["codes"], scales=p["scales"])

    for i in range(max(1, args.warmup)):
        step(i % R)
    torch.cuda.synchronize()

    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(R):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step(r)
        graphs.append(gr)
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        graphs[i % R].replay()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] graph steps: {ms_per_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    n = len(pts)
    evs = [(hip.event(), hip.event()) for _ in range(args.steps * n)]
    for i in range(args.steps):
        for j, p in enumerate(pts):
            hq._check(L.hq_time_next_launch(*evs[i * n + j]))
            hq.quantize_per_token(p["xs"][i % R], p["out"], codes=p["codes"], scales=p["scales"])
    torch.cuda.synchronize()
    per_point, tot = [], 0.0
    for j, p in enumerate(pts):
        ms = [hip.elapsed_ms(*evs[i * n + j]) for i in range(args.steps)]
        tot += float(np.sum(ms))
        us = float(np.mean(ms)) * 1e3
        per_point.append({"M": p["M"], "K": QUANT_K, "out": p["out"], "kernel_us": round(us, 3),
                          "GBps": round(p["bytes"] / (us * 1e-6) / 1e9, 1),
                          "hbm_frac": round(p["bytes"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    mean_us = tot / (args.steps * n) * 1e3
    achieved = step_bytes / n / (mean_us * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu:
        # the CPU oracle leg: a spot check of the last timed launches' output, then its timing
        from oracle import quant as QZ

        for p in pts[-2:]:
            ref_c, ref_s = QZ.quantize_rows(p["xs"][(args.steps - 1) % R].float().cpu().numpy(), p["out"])
            if not (np.array_equal(p["codes"].cpu().numpy(), ref_c)
                    and np.array_equal(p["scales"].cpu().numpy(), ref_s)):
                raise SystemExit(f"bench: quantiser output check failed (M={p['M']} {p['out']})")
        print("[bench] spot check against the oracle ok (codes and scales bit-exact); timing the CPU oracle",
              file=sys.stderr, flush=True)
        done, secs, runs = 0, 0.0, 0
        while secs < args.cpu_budget:
            for M in QUANT_M:
                x = torch.randn((M, QUANT_K), generator=torch.Generator().manual_seed(M)).to(torch.bfloat16)
                xf = x.float().numpy()
                for out in ("fp8", "int8"):
                    t0 = time.perf_counter()
                    QZ.quantize_rows(xf, out)
                    secs += time.perf_counter() - t0
                    done += quant_bytes(M, QUANT_K)
                    runs += 1
        cpu = {"value": done / secs / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{runs} oracle runs over the 8 points of the workload (numpy float32 division, "
                         f"float64 rounding to the code grid), {secs:.1f} s total, single-threaded numpy"}

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": QUANT_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": QUANT_WORKLOAD, "launches_per_step": n, "step_bytes": step_bytes,
                   "input_rotations": R, "timing": "HIP graph replay per step; kernel durations from "
                                                   "dispatch-bracketing HIP events"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "hq::quantize_rows_kernel", "mean_kernel_us": round(mean_us, 3),
                     "mean_algorithmic_bytes": int(step_bytes / n)},
        "cpu_baseline": cpu,
        "points": per_point,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotations", type=int, default=4)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", choices=("decode", "quant"), default="decode",
                    help="decode: the dense W4A16 decode sweep (default); quant: the per-token quantiser")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested); the sharded "
              "form is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    if args.workload == "quant":
        run_quant(args)
        return

    import bit_quantized_gemm_repack_amd as hq

    dev = torch.device("cuda:0")
    hip = Hip()
    L = hq.lib()
    print(f"[bench] preparing {len(SWEEP_M) * len(SWEEP_NK)} points x {args.rotations} rotations", file=sys.stderr,
          flush=True)
    points, shapes = make_points(dev, args.rotations)
    R = args.rotations
    step_bytes = sum(p["bytes"] for p in points)
    step_flops = sum(p["flops"] for p in points)

    # eager warm-up (also allocates nothing new: outputs / workspaces exist)
    for i in range(max(1, args.warmup)):
        run_step(points, i % R)
    torch.cuda.synchronize()

    # --- graphs: one per rotation -------------------------------------------
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_step(points, 0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_step(points, r)
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        graphs[i % R].replay()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    ms_per_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] graph steps: {ms_per_step * 1e3:.1f} us/step (wall {wall_ms / args.steps * 1e3:.1f})",
          file=sys.stderr, flush=True)

    # --- per-kernel durations (events around each dispatch) ------------------
    n = len(points)
    evs = [(hip.event(), hip.event()) for _ in range(args.steps * n)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        r = i % R
        for j, p in enumerate(points):
            st, en = evs[i * n + j]
            hq._check(L.hq_time_next_launch(st, en))
            w, meta = p["copies"][r]
            p["plan"].gemm(p["a"], w, meta, out=p["out"], ws=p["ws"])
    torch.cuda.synchronize()
    per_point = []
    tot_k_ms = 0.0
    for j, p in enumerate(points):
        ms = [hip.elapsed_ms(*evs[i * n + j]) for i in range(args.steps)]
        us = float(np.mean(ms)) * 1e3
        tot_k_ms += float(np.sum(ms))
        gbs = p["bytes"] / (us * 1e-6) / 1e9
        per_point.append({"M": p["M"], "N": p["N"], "K": p["K"], "kernel_us": round(us, 3),
                          "kernel_us_p10": round(float(np.percentile(ms, 10)) * 1e3, 3),
                          "kernel_us_p90": round(float(np.percentile(ms, 90)) * 1e3, 3),
                          "GBps": round(gbs, 1), "TFLOPS": round(p["flops"] / (us * 1e-6) / 1e12, 2),
                          "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                          "plan": p["plan"].describe(p["M"])})
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    launches = args.steps * n
    mean_kernel_us = tot_k_ms / launches * 1e3
    mean_bytes = step_bytes / n
    achieved = mean_bytes / (mean_kernel_us * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu:
        # the CPU oracle leg: a spot check of the timed launches' output, then its timing
        max_ratio = check_point(points, shapes)
        print(f"[bench] spot check against the oracle ok (max err/tau {max_ratio:.3g}); timing the CPU oracle",
              file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.cpu_budget)
        cpu["spot_check_max_err_over_tau"] = round(max_ratio, 4)

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "launches_per_step": n, "step_bytes": step_bytes,
                   "step_flops": step_flops, "tflops_per_step_time": round(step_flops / (ms_per_step * 1e-3) / 1e12, 3),
                   "weight_pool_rotations": R, "timing": "HIP graph replay per step; kernel durations from "
                                                         "dispatch-bracketing HIP events"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "hq_gemm calls of the sweep: hq::qgemm_skinny / hq::qgemm_tiled "
                               "(+ hq::splitk_reduce_kernel where K is split)",
                     "mean_kernel_us": round(mean_kernel_us, 3), "mean_algorithmic_bytes": int(mean_bytes)},
        "cpu_baseline": cpu,
        "points": per_point,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
