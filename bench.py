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
  * ceilings: what a plain streaming read (the library's probe, no
    arithmetic) attains on this GPU: over 1 GiB, and over each point's packed
    weights from the same rotating pool, with the GEMMs' achieved bandwidth
    as a fraction of the latter.

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


# sources of the kernels a decode-sweep call runs (GEMM, split-K reduce, their
# shared headers and launch helper); the plan strings cover the host heuristic
DECODE_KERNEL_SOURCES = ("csrc/qgemm_skinny.hip", "csrc/qgemm_skinny_kernel.h", "csrc/qgemm_tiled.hip",
                         "csrc/qgemm_tiled_kernel.h",
                         "csrc/splitk_reduce.hip", "csrc/device_common.h", "csrc/hq_internal.h", "csrc/launch.h",
                         "build.py")


def kernel_source_hash():
    """sha256 over the sources (and build flags) of the decode-sweep kernels."""
    import hashlib

    pkg = os.path.join(ROOT, "bit_quantized_gemm_repack_amd")
    h = hashlib.sha256()
    for name in DECODE_KERNEL_SOURCES:
        h.update(name.encode())
        with open(os.path.join(pkg, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(plans=None):
    """HBM bytes per call from the counter summary, if it was taken on these
    kernel sources and (when given) with these per-point plans."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    if plans is not None and [q.get("plan") for q in t.get("points", [])] != list(plans):
        return None
    return t.get("hbm_bytes_per_call")


def write_profiles(run_dir):
    """Summaries under profiles/ from the rocprofv3 outputs of the decode bench
    in run_dir (CPU only; the GPU commands are listed in the files written):
      prof_bench/bench_kernel_{stats,trace}.csv  --kernel-trace --stats run
      pmc_fetch/f_counter_collection.csv         --pmc FETCH_SIZE run
      pmc_write/w_counter_collection.csv         --pmc WRITE_SIZE run
      bench.json                                 a default bench run (last line)."""
    import collections
    import csv

    def rows(path):
        with open(os.path.join(run_dir, path)) as f:
            return list(csv.DictReader(f))

    n = len(SWEEP_M) * len(SWEEP_NK)
    pts = [(M, N, K) for M in SWEEP_M for (N, K) in SWEEP_NK]
    with open(os.path.join(run_dir, "bench.json")) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    plans = [p["plan"] for p in b["points"]]

    # --- traffic: FETCH_SIZE / WRITE_SIZE per call (GEMM + its reduce) -------
    fetch = sorted(rows("pmc_fetch/f_counter_collection.csv"), key=lambda r: int(r["Dispatch_Id"]))
    write = rows("pmc_write/w_counter_collection.csv")
    wr = {r["Dispatch_Id"]: float(r["Counter_Value"]) for r in write}
    # calibration: the runtime's copy kernels (the weight-pool clones) read what they write
    cf = [(float(r["Counter_Value"]), wr[r["Dispatch_Id"]]) for r in fetch if "copyBuffer" in r["Kernel_Name"]]
    fetch_scale = sum(w for _, w in cf) / sum(f for f, _ in cf)
    calls, cur = [], None
    for r in fetch:
        k = r["Kernel_Name"]
        if "qgemm" in k:
            cur = {"kernel": k.split("(")[0], "fetch": float(r["Counter_Value"]), "write": wr[r["Dispatch_Id"]]}
            calls.append(cur)
        elif "splitk_reduce" in k and cur is not None:
            cur["fetch"] += float(r["Counter_Value"])
            cur["write"] += wr[r["Dispatch_Id"]]
            cur["reduce"] = True
    per = collections.defaultdict(list)
    for i, c in enumerate(calls):
        per[i % n].append(c)
    tpoints, tot = [], 0.0
    for j in range(n):
        cs = per[j]
        fb = sum(c["fetch"] for c in cs) / len(cs) * 1024 * fetch_scale
        wb = sum(c["write"] for c in cs) / len(cs) * 1024
        M, N, K = pts[j]
        alg = algo_bytes(M, N, K)
        tpoints.append(dict(M=M, N=N, K=K, kernel=cs[0]["kernel"], reduce=bool(cs[0].get("reduce")),
                            hbm_read=int(fb), hbm_write=int(wb), algorithmic=alg, ratio=round((fb + wb) / alg, 3),
                            plan=plans[j]))
        tot += fb + wb
    cmd = "cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <repo>/gpurun_out/{d} -o {o} -- " \
          "python3 <repo>/bench.py --steps 3 --warmup 1 --no-cpu --no-extra"
    traffic = {"source_sha256": kernel_source_hash(), "hbm_bytes_per_call": int(tot / n),
               "algorithmic_bytes_per_call": int(sum(algo_bytes(*p) for p in pts) / n),
               "fetch_scale": round(fetch_scale, 4), "write_scale": 1.0,
               "calibration": "FETCH_SIZE (KiB per dispatch) scaled by written/fetched of the runtime's copy kernels "
                              "in the same runs (a plain copy reads what it writes); WRITE_SIZE taken as is",
               "commands": [cmd.format(c="FETCH_SIZE", d="pmc_fetch", o="f"),
                            cmd.format(c="WRITE_SIZE", d="pmc_write", o="w"),
                            "python3 bench.py --write-profiles gpurun_out   (this summary, on the CPU)"],
               "points": tpoints}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(traffic, f, indent=1)

    # --- kernel trace: per-kernel stats and per-call durations ---------------
    stats = rows("prof_bench/bench_kernel_stats.csv")
    trace = sorted(rows("prof_bench/bench_kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    calls, cur = [], None
    for r in trace:
        k = r["Kernel_Name"]
        st, en = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if "qgemm" in k:
            cur = [st, en]
            calls.append(cur)
        elif "splitk_reduce" in k and cur is not None:
            cur[1] = en
    dur = [(c[1] - c[0]) / 1e3 for c in calls]
    timed = dur[-20 * n:]
    graph = dur[-40 * n:-20 * n]
    mean_timed = sum(timed) / len(timed)
    L = ["# qgemm -- dense W4A16 decode sweep, bf16, uint4 zero points (skinny / tiled + split-K reduce)", "",
         "Workload: M in {1,4,16,64} x (N,K) in {(4096,4096),(14336,4096),(4096,14336)}, group 128, bf16 scales,",
         "uint4 zero points, bf16 output; every call reads its own copy of the weights from a rotating pool (> 1 GB).",
         "", "Kernel trace (from the repository root on the GPU host):", "", "```",
         "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <repo>/gpurun_out/prof_bench -o bench -- \\",
         "    python3 <repo>/bench.py --steps 20 --warmup 5 --no-cpu --no-extra",
         "python3 bench.py --write-profiles gpurun_out      # this file and the traffic summary, on the CPU", "```", "",
         "`bench_kernel_stats.csv`, library kernels (every dispatch of the run: eager warm-up, graph replays, "
         "event-timed pass):", "", "| kernel | calls | total ns | average ns | min ns | max ns |", "|---|---|---|---|---|---|"]
    for r in stats:
        if "hq::" in r["Name"]:
            L.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {r['TotalDurationNs']} | {float(r['AverageNs']):.0f} | "
                     f"{r['MinNs']} | {r['MaxNs']} |")
    L += ["", f"hq_gemm calls in the trace (GEMM dispatch start to the end of its split-K reduce, where there is one): "
              f"the traced run's event-timed pass (its last {len(timed)} calls) averages {mean_timed:.2f} us per call, "
              f"its graph replays {sum(graph) / len(graph):.2f} us, all {len(calls)} calls {sum(dur) / len(dur):.2f} us "
              f"(the first passes run on cold caches and workspaces).  The default run below gives "
              f"{b['roofline']['mean_call_us']:.2f} us per call over its graph-replayed step (the roofline's figure, "
              f"{100 * (b['roofline']['mean_call_us'] / (sum(graph) / len(graph)) - 1):+.1f} % against the traced "
              f"graph replays, which carry the profiler's overhead) and "
              f"{sum(q['kernel_us'] for q in b['points']) / len(b['points']):.2f} us per call from its "
              f"dispatch-bracketing events.", "",
          f"Bench line (default `python3 bench.py`): {b['value']} GB/s over the step ({b['ms_per_step'] * 1e3:.1f} us "
          f"per step of {n} graph-replayed calls); roofline achieved {b['roofline']['achieved']} GB/s = "
          f"{100 * b['roofline']['frac']:.1f} % of 8 TB/s; CPU oracle {b['cpu_baseline']['value']:.3f} GB/s on "
          f"{b['cpu_baseline']['cores']} BLAS threads.", "",
          "| M | N | K | us | GB/s | % of 8 TB/s | HBM bytes / algorithmic | plan |", "|---|---|---|---|---|---|---|---|"]
    for p, t in zip(b["points"], tpoints):
        L.append(f"| {p['M']} | {p['N']} | {p['K']} | {p['kernel_us']:.2f} | {p['GBps']:.0f} | "
                 f"{100 * p['hbm_frac']:.1f} | {t['ratio']:.2f} | {p['plan']} |")
    L += ["", "Per point, the bench's events against the trace (mean over the traced run's event-timed pass and its "
              "graph replays; the profiler widens the gap between a split-K GEMM and its reduce):", "",
          "| M | N | K | bench events us | trace, timed pass us | trace, graph replays us |", "|---|---|---|---|---|---|"]
    for j, p in enumerate(b["points"]):
        tj = [timed[i] for i in range(j, len(timed), n)]
        gj = [graph[i] for i in range(j, len(graph), n)]
        L.append(f"| {p['M']} | {p['N']} | {p['K']} | {p['kernel_us']:.2f} | {sum(tj) / len(tj):.2f} | "
                 f"{sum(gj) / len(gj):.2f} |")
    L += ["", f"HBM traffic per call (`qgemm_decode_sweep_traffic.json`): FETCH_SIZE and WRITE_SIZE from two `--pmc` "
              f"runs of the same bench (commands in that file), FETCH scaled by {traffic['fetch_scale']} (the copy "
              f"kernels' written/fetched ratio), WRITE by 1.0: {traffic['hbm_bytes_per_call'] / 1e6:.2f} MB per call "
              f"against {traffic['algorithmic_bytes_per_call'] / 1e6:.2f} MB algorithmic."]
    with open(os.path.join(ROOT, "profiles", "qgemm_decode_sweep_w4a16_bf16.md"), "w") as f:
        f.write("\n".join(L) + "\n")
    print(f"wrote {TRAFFIC_FILE} and profiles/qgemm_decode_sweep_w4a16_bf16.md")
    _write_workload_profiles(run_dir, rows)


_WORKLOAD_PROFILES = {
    "quant": ("quantize_rows_per_token_k7168.md", "per-token activation quantiser, x bf16 [M, 7168], "
              "M in {1,16,128,1024}, fp8 and int8 codes"),
    "prefill": ("qgemm_tiled_prefill_w4a16_f16.md", "dense W4A16 prefill, M in {1024,4096}, N = K = 8192, fp16"),
    "w4a8": ("qgemm_w4a8_mxfp4_int8_n4096_k7168.md", "dense W4A8, M in {1,16,128,1024}, N = 4096, K = 7168, "
             "MXFP4 x fp8 and INT4 x int8"),
    "w4a4": ("qgemm_w4a4_mxfp4_n4096_k7168.md", "dense W4A4, M in {1,16,128,1024}, N = 4096, K = 7168, "
             "MXFP4 x MXFP4"),
    "w8a16": ("qgemm_w8a16_bf16_n4096_k4096.md", "dense W8A16, M in {1,16,64,1024}, N = K = 4096, bf16"),
    "w2a16": ("qgemm_w2a16_bf16_n4096_k4096.md", "dense W2A16, M in {1,16,64,1024}, N = K = 4096, bf16"),
    "w3a16": ("qgemm_w3a16_bf16_n4096_k4096.md", "dense W3A16, M in {1,16,64,1024}, N = K = 4096, bf16"),
    "mxint4": ("qgemm_w4a16_mxint4_bf16_n4096_k4096.md", "dense W4A16-MXINT4, M in {1,16,64,1024}, N = K = 4096, "
               "bf16"),
    "nvfp4": ("qgemm_w4a16_nvfp4_bf16_n4096_k4096.md", "dense W4A16-NVFP4, M in {1,16,64,1024}, N = K = 4096, "
              "bf16"),
    "moe": ("moe_layer_e256_top8_h7168_i256.md", "MoE layer, 256 experts, top-8, hidden 7168, intermediate 256, "
            "T in {1,4,8,32,512,4096} (aligned) and {1,4,8,32} (by slot), bf16 and fp8 activations"),
}


def _write_workload_profiles(run_dir, rows):
    """profiles/<kernel>_<workload>.md for each workload traced in run_dir:
    prof_<w>/<w>_kernel_stats.csv (--kernel-trace --stats) and, if present,
    bench_<w>.log (the workload's bench line)."""
    for w, (fname, what) in _WORKLOAD_PROFILES.items():
        path = os.path.join(run_dir, f"prof_{w}", f"{w}_kernel_stats.csv")
        if not os.path.exists(path):
            continue
        stats = rows(f"prof_{w}/{w}_kernel_stats.csv")
        L = [f"# {what}", "", "Kernel trace (from the repository root on the GPU host):", "", "```",
             f"cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <repo>/gpurun_out/prof_{w} -o {w} -- \\",
             f"    python3 <repo>/bench.py --workload {w} --steps 10 --warmup 2 --no-cpu",
             "python3 bench.py --write-profiles gpurun_out      # this summary, on the CPU", "```", "",
             f"`{w}_kernel_stats.csv`, library kernels (every dispatch of the run: eager warm-up, graph replays, "
             "event-timed pass; averages mix the workload's points where one kernel serves several):", "",
             "| kernel | calls | total ns | average ns | min ns | max ns |", "|---|---|---|---|---|---|"]
        for r in stats:
            if "hq::" in r["Name"]:
                L.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {r['TotalDurationNs']} | {float(r['AverageNs']):.0f} | "
                         f"{r['MinNs']} | {r['MaxNs']} |")
        log = os.path.join(run_dir, f"bench_{w}.log")
        if os.path.exists(log):
            with open(log) as f:
                lines = [x for x in f if x.startswith("{")]
            if lines:
                b = json.loads(lines[-1])
                cmd = f"python3 bench.py --workload {w}" + (" --steps 20 --warmup 3 --cpu-budget 8" if w != "quant"
                                                             else " --cpu-budget 5")
                L += ["", f"Bench line (`{cmd}`): value {b['value']} {b['unit']} ({b['ms_per_step'] * 1e3:.1f} us per "
                          f"step); roofline {json.dumps(b['roofline'])}; CPU oracle "
                          f"{b['cpu_baseline']['value']:.4g} {b['cpu_baseline']['unit']} "
                          f"({b['cpu_baseline']['sample']}).", ""]
                if w == "quant":
                    L += ["| M | codes | us | GB/s | % of 8 TB/s |", "|---|---|---|---|---|"]
                    for p in b["points"]:
                        L.append(f"| {p['M']} | {p['out']} | {p['kernel_us']:.2f} | {p['GBps']:.0f} | "
                                 f"{100 * p['hbm_frac']:.1f} |")
                else:
                    L += ["Per point: one graph over the point's whole weight pool, the mean pass (us).", "",
                          "| point | us | GB/s | TFLOP/s | bound | % of bound | plan |",
                          "|---|---|---|---|---|---|---|"]
                    for p in b["points"]:
                        L.append(f"| {p['point']} | {p['us']:.1f} | {p['GBps']:.0f} | {p['TFLOPS']:.1f} | "
                                 f"{p['bound']} | {100 * p['roofline_frac']:.1f} | {p['plan']} |")
        with open(os.path.join(ROOT, "profiles", fname), "w") as f:
            f.write("\n".join(L) + "\n")
        print(f"wrote profiles/{fname}")
    _write_counter_profiles(run_dir, rows)


# Two SQ counter passes of a workload's bench (rocprofv3 collects at most
# eight SQ counters per pass): sq_<w>_1 and sq_<w>_2 in the run directory.
SQ_PASSES = ("SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY "
             "SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU",
             "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_VMEM_RD SQ_INST_LEVEL_VMEM "
             "SQ_ACTIVE_INST_LDS SQ_WAVES")
# memory side, for the weight-streaming decode kernels (a third pass where it was taken)
MEM_PASS = ("TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_PENDING_STALL_CYCLES_sum "
            "TCP_READ_TAGCONFLICT_STALL_CYCLES_sum TA_BUSY_avr TA_ADDR_STALLED_BY_TC_CYCLES_sum TCC_HIT_sum TCC_MISS_sum "
            "GRBM_GUI_ACTIVE SQ_WAVES")
# workloads whose counter passes run with other flags than the per-workload bench
_COUNTER_ONLY = {"decode": ("qgemm_decode_sweep_w4a16_bf16.md", "dense W4A16 decode sweep, bf16, uint4 zero points, "
                            "M in {1,4,16,64} x (N,K) in {(4096,4096),(14336,4096),(4096,14336)}", "--no-extra")}


def _write_counter_profiles(run_dir, rows):
    """profiles/<workload file>_sq_counters.md: per library kernel, the mean of
    each SQ counter over its dispatches, and the derived figures."""
    import collections

    todo = {w: (fname, what, "") for w, (fname, what) in _WORKLOAD_PROFILES.items()}
    todo.update(_COUNTER_ONLY)
    for w, (fname, what, flags) in todo.items():
        paths = [os.path.join(run_dir, f"sq_{w}_{i}", f"c_counter_collection.csv") for i in (1, 2)]
        if not all(os.path.exists(x) for x in paths):
            continue
        mem = os.path.exists(os.path.join(run_dir, f"sq_{w}_3", "c_counter_collection.csv"))
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for i in (1, 2):
            for r in rows(f"sq_{w}_{i}/c_counter_collection.csv"):
                k = r["Kernel_Name"].split("(")[0]
                if "hq::" in k:
                    agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        magg = collections.defaultdict(lambda: collections.defaultdict(list))
        if mem:
            for r in rows(f"sq_{w}_3/c_counter_collection.csv"):
                k = r["Kernel_Name"].split("(")[0]
                if "hq::" in k:
                    magg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        L = [f"# SQ counters: {what}", "", f"{3 if mem else 2} counter passes of the workload's bench (from the "
             "repository root on the GPU host), then this summary on the CPU:", "", "```"]
        extra = f" {flags}" if flags else ""
        for i, c in enumerate(SQ_PASSES + ((MEM_PASS,) if mem else ()), 1):
            L.append(f"cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <repo>/gpurun_out/sq_{w}_{i} -o c -- "
                     f"python3 <repo>/bench.py --workload {w} --steps 3 --warmup 1 --no-cpu{extra}")
        means = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in agg.items()}

        def busy_ratio(m):
            return m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / max(m.get("SQ_BUSY_CYCLES", 0.0), 1.0)

        # the register-only matrix-core probe of each operand type, from the same run
        probe = {int(k.split("<")[1].split(">")[0]): busy_ratio(m) for k, m in means.items()
                 if "mfma_peak_kernel<" in k}
        # kernel format (first template argument) -> probe type (f16 0, bf16 1, fp8 2, fp8 x fp4 3, fp4 4, int8 5)
        fmt_probe = {0: 0, 1: 1, 2: 5, 3: 2, 4: 3, 5: 4}
        L += ["python3 bench.py --write-profiles gpurun_out", "```", "",
              "Per kernel, the means over its dispatches, as unit-free ratios: VALU instructions per MFMA; LDS bank "
              "conflicts per LDS instruction; the share of the waves' time spent waiting (SQ_WAIT_ANY / "
              "SQ_WAVE_CYCLES) and issuing (SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES); and the matrix cores' busy time "
              "relative to the SQ's busy time (SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CYCLES), also as a fraction of the "
              "same ratio for the library's register-only matrix-core probe of the kernel's operand type in the "
              "same run (`mfma_peak_kernel<type>`, types f16 0, bf16 1, fp8 2, fp8 x fp4 3, fp4 4, int8 5).", "",
              "| kernel | dispatches | waves | MFMA instr | VALU / MFMA | bank conflicts / LDS instr | waiting share | "
              "issuing share | MFMA busy / SQ busy | of the probe's |",
              "|---|---|---|---|---|---|---|---|---|---|"]
        for k, m in sorted(means.items()):
            n = max(len(v) for v in agg[k].values())
            wc = max(m.get("SQ_WAVE_CYCLES", 0.0), 1.0)
            mf = m.get("SQ_INSTS_MFMA", 0.0)
            vpm = f"{m.get('SQ_INSTS_VALU', 0.0) / mf:.2f}" if mf else "-"
            bc = m.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(m.get("SQ_INSTS_LDS", 0.0), 1.0)
            br = busy_ratio(m)
            rel = "-"
            if ("qgemm" in k or "smallk" in k) and "<" in k:
                fmt = int(k.split("<")[1].split(",")[0])
                ptype = fmt_probe.get(fmt, 0 if fmt % 2 == 0 else 1)
                if probe.get(ptype):
                    rel = f"{br / probe[ptype]:.2f}"
            L.append(f"| `{k[:80]}` | {n} | {m.get('SQ_WAVES', 0.0):.0f} | {mf:.0f} | {vpm} | {bc:.3f} | "
                     f"{m.get('SQ_WAIT_ANY', 0.0) / wc:.2f} | {m.get('SQ_ACTIVE_INST_ANY', 0.0) / wc:.2f} | {br:.3f} | "
                     f"{rel} |")
        if mem:
            L += _memory_table(magg, run_dir, w)
        out = fname.replace(".md", "_sq_counters.md")
        with open(os.path.join(ROOT, "profiles", out), "w") as f:
            f.write("\n".join(L) + "\n")
        print(f"wrote profiles/{out}")


def _memory_table(magg, run_dir, w):
    """The memory-side pass, per kernel: L1 -> L2 read latency, L2 hit rate,
    and the shares of the texture units' busy time lost to cache stalls, with
    the plain streaming read of the same run as the reference."""
    cus = 256
    try:
        import csv
        with open(os.path.join(run_dir, f"sq_{w}_3", "c_agent_info.csv")) as f:
            for r in csv.DictReader(f):
                if int(r.get("cu_count", 0) or 0) > 0:
                    cus = int(r["cu_count"])
    except (OSError, ValueError, KeyError):
        pass
    L = ["", "Memory-side pass (third command), per kernel, the means over its dispatches:",
         "* L1 -> L2 read latency: TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ, cycles per read request;",
         "* L2 hit rate: TCC_HIT / (TCC_HIT + TCC_MISS);",
         f"* as shares of the texture units' busy cycles ({cus} x TA_BUSY_avr, one unit per CU): cycles the L1 "
         "stalled with its pending-miss tracking full (TCP_PENDING_STALL_CYCLES), on read tag conflicts "
         "(TCP_READ_TAGCONFLICT_STALL_CYCLES), and cycles the address path waited on the L1 "
         "(TA_ADDR_STALLED_BY_TC_CYCLES);",
         "* TA busy: TA_BUSY_avr / GRBM_GUI_ACTIVE, relative to the same ratio of the plain streaming read "
         "(`stream_read_kernel`) in the same run.", "",
         "| kernel | dispatches | L1 -> L2 latency (cycles) | L2 hit rate | pending-miss stall | tag-conflict stall | "
         "address stalled by L1 | TA busy vs the plain read |", "|---|---|---|---|---|---|---|---|"]
    means = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in magg.items()}

    def ta_busy(m):
        return m.get("TA_BUSY_avr", 0.0) / max(m.get("GRBM_GUI_ACTIVE", 0.0), 1.0)

    ref = next((ta_busy(m) for k, m in means.items() if "stream_read_kernel" in k), 0.0)
    for k, m in sorted(means.items()):
        n = max(len(v) for v in magg[k].values())
        lat = m.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) / max(m.get("TCP_TCC_READ_REQ_sum", 0.0), 1.0)
        h, mi = m.get("TCC_HIT_sum", 0.0), m.get("TCC_MISS_sum", 0.0)
        hit = f"{h / (h + mi):.2f}" if h + mi > 0 else "-"
        tb = max(cus * m.get("TA_BUSY_avr", 0.0), 1.0)
        rel = f"{ta_busy(m) / ref:.2f}" if ref > 0 else "-"
        L.append(f"| `{k[:80]}` | {n} | {lat:.0f} | {hit} | {m.get('TCP_PENDING_STALL_CYCLES_sum', 0.0) / tb:.2f} | "
                 f"{m.get('TCP_READ_TAGCONFLICT_STALL_CYCLES_sum', 0.0) / tb:.2f} | "
                 f"{m.get('TA_ADDR_STALLED_BY_TC_CYCLES_sum', 0.0) / tb:.2f} | {rel} |")
    return L


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


def make_points(dev, rotations, autotune=False):
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
            if autotune:  # measured choice for this m in place of the heuristic (weights from HBM)
                r = plan.autotune(a, copies[0][0], copies[0][1], reps=10, flush_bytes=512 << 20)
                print(f"[bench] autotune M={M} N={N} K={K}: {r['current_us']:.2f} -> {r['best_us']:.2f} us "
                      f"{r['tuning']}", file=sys.stderr, flush=True)
            ws = plan.workspace(M, dev)
            points.append(dict(M=M, N=N, K=K, plan=plan, a=a, copies=copies, out=out, ws=ws,
                               bytes=algo_bytes(M, N, K), flops=algo_flops(M, N, K)))
    torch.cuda.synchronize()
    return points, shapes


def run_step(points, r):
    for p in points:
        w, meta = p["copies"][r]
        p["plan"].gemm(p["a"], w, meta, out=p["out"], ws=p["ws"])


def check_points(points, shapes):
    """Every point's last timed output against the CPU oracle: all rows of
    each point (the M = 64 oracle result of a shape covers its smaller M, whose
    activations are its first rows).  Returns the largest err / tau and the
    fraction of outputs within the literal tau (without the output format's
    half ulp)."""
    from oracle import gemm as og

    refs = {}
    worst, lit_ok, total = 0.0, 0, 0
    for p in points:
        key = (p["N"], p["K"])
        if key not in refs:
            d = shapes[key]["data"]
            refs[key] = og.gemm_w4a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(),
                                      d["zeros"], out_fmt="bf16")
        ref = refs[key]
        M = p["M"]
        ok, lit, ratio = og.check(p["out"].double().cpu().numpy(), ref["c64"][:M], ref["tau"][:M], "bf16")
        if not ok.all():
            raise SystemExit(f"bench: output check failed at M={M} N={p['N']} K={p['K']} "
                             f"({int((~ok).sum())} outputs, max err/tau {ratio.max():.3g})")
        worst = max(worst, float(ratio.max()))
        lit_ok += int(lit.sum())
        total += lit.size
    return worst, lit_ok / total, total


class GpuStateSampler:
    """The GPU's shader clock and power, read in this process from the amdgpu
    driver's sysfs files (pp_dpm_sclk: the level marked '*' is the current
    one; hwmon power1_average or power1_input, microwatts) by a thread that
    samples every `period` seconds while the timed replays run.  No child
    process is started.  The card is the one whose PCI address matches
    torch's device 0; None where the files are not readable."""

    def __init__(self, period=0.001):
        import glob
        import threading

        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        self.card = None
        try:
            pr = torch.cuda.get_device_properties(0)
            want = (int(pr.pci_domain_id), int(pr.pci_bus_id), int(pr.pci_device_id))
        except Exception:  # pragma: no cover
            want = None
        for dev_dir in sorted(glob.glob("/sys/class/drm/card*/device")):
            try:
                bdf = os.path.basename(os.path.realpath(dev_dir))  # dddd:bb:dd.f
                dom, bus, rest = bdf.split(":")
                key = (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16))
            except ValueError:
                continue
            if (want is None or key == want) and os.path.exists(os.path.join(dev_dir, "pp_dpm_sclk")):
                self.card = dev_dir
                break
        self.power_file = None
        if self.card:
            for name in ("power1_average", "power1_input"):
                hits = sorted(glob.glob(os.path.join(self.card, "hwmon", "hwmon*", name)))
                if hits:
                    self.power_file = hits[0]
                    break

    def _read(self):
        clk = pw = None
        try:
            with open(os.path.join(self.card, "pp_dpm_sclk")) as f:
                for line in f:
                    if "*" in line:
                        clk = float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            pass
        if self.power_file:
            try:
                with open(self.power_file) as f:
                    pw = int(f.read().strip()) / 1e6
            except (OSError, ValueError):
                pass
        return clk, pw

    def _run(self):
        while not self._stop.is_set():
            self.samples.append(self._read())
            self._stop.wait(self.period)

    def __enter__(self):
        import threading

        if self.card:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self):
        if not self.card:
            return None
        clks = [c for c, _ in self.samples if c is not None]
        pws = [w for _, w in self.samples if w is not None]
        return {"gfx_clk_mhz_mean": round(float(np.mean(clks)), 1) if clks else None,
                "gfx_clk_mhz_min": min(clks) if clks else None, "gfx_clk_mhz_max": max(clks) if clks else None,
                "power_w_mean": round(float(np.mean(pws)), 1) if pws else None, "samples": len(self.samples),
                "source": f"{self.card}/pp_dpm_sclk and {self.power_file}",
                "when": "sampled in-process every ~1 ms during the timed graph replays"}


def mfma_ceilings(hip, L, dev):
    """Sustained matrix-core rate (TFLOP/s or TOP/s) of every operand type the
    GEMMs use, from the library's register-only probe (hq_mfma_peak): median of
    five launches of 1024 workgroups, timed with dispatch-bracketing events."""
    import bit_quantized_gemm_repack_amd as hq

    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    kinds = {"f16": hq.PEAK_F16, "bf16": hq.PEAK_BF16, "fp8": hq.PEAK_FP8, "fp8_fp4": hq.PEAK_FP8_FP4,
             "fp4": hq.PEAK_FP4, "int8": hq.PEAK_INT8}
    out = {}
    for name, k in kinds.items():
        hq.mfma_peak(k, sink, 1024, 200)  # warm-up (clock ramp)
        rates = []
        for _ in range(5):
            a, b = hip.event(), hip.event()
            hq._check(L.hq_time_next_launch(a, b))
            fl = hq.mfma_peak(k, sink, 1024, 2000)
            torch.cuda.synchronize()
            rates.append(fl / (hip.elapsed_ms(a, b) * 1e-3) / 1e12)
            hip.destroy(a)
            hip.destroy(b)
        out[name] = round(float(np.median(rates)), 1)
    return out


def measure_ceilings(points, hip, L, R, steps):
    """Attainable-bandwidth references measured with the library's plain
    streaming-read probe (16-byte loads, no arithmetic): a 1 GiB read, and a
    read of each point's packed weights (the bulk of its bytes) from the same
    rotating pool, timed with the same dispatch-bracketing events as the
    GEMMs.  The best of three grid sizes is kept."""
    import bit_quantized_gemm_repack_amd as hq

    dev = points[0]["a"].device
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def timed_read(buf, nbytes, wgs, reps):
        evs = [(hip.event(), hip.event()) for _ in range(reps)]
        for i in range(reps):
            hq._check(L.hq_time_next_launch(*evs[i]))
            hq.stream_read(buf[i % len(buf)], sink, wgs, nbytes)
        torch.cuda.synchronize()
        ms = sorted(hip.elapsed_ms(a, b) for a, b in evs)
        for a, b in evs:
            hip.destroy(a)
            hip.destroy(b)
        return ms[len(ms) // 2] * 1e3

    big = [torch.empty(1 << 30, dtype=torch.uint8, device=dev)]
    big_us = min(timed_read(big, 1 << 30, w, 10) for w in (1024, 2048, 4096))
    del big
    point_us = []
    for p in points:
        bufs = [c[0] for c in p["copies"]]
        nb = bufs[0].numel() * bufs[0].element_size() // 16 * 16
        point_us.append(round(min(timed_read(bufs, nb, w, max(8, min(steps, 40))) for w in (512, 1024, 2048)), 3))
    wbytes = sum(c["copies"][0][0].numel() * c["copies"][0][0].element_size() // 16 * 16 for c in points)
    return {"stream_read_1GiB_GBps": round((1 << 30) / (big_us * 1e-6) / 1e9, 1),
            "same_bytes_read_GBps": round(wbytes / (sum(point_us) * 1e-6) / 1e9, 1),
            "what": "plain streaming reads by the library's probe: 1 GiB, and each point's packed weights "
                    "(the bulk of its bytes) from the same rotating pool; roofline.achieved / same_bytes_read_GBps "
                    "= frac_of_same_bytes_read",
            "point_read_us": point_us}


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
    for gr in graphs:  # a graph's first launch uploads it: once each, before the warm-up steps
        gr.replay()
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with GpuStateSampler() as smp:
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
        "gpu_state": smp.summary(),
        "points": per_point,
    }
    print(json.dumps(line), flush=True)


# ----------------------------------------------------------------------------
# Further workloads (non-default): each point is a list of library calls; a
# point's time is the sum of its calls' durations (dispatch-bracketing events),
# its roofline t_roof = max(flops / MFMA peak of its dtype, bytes / 8 TB/s).
# ----------------------------------------------------------------------------
FP16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0


def _prefill_points(dev, Ms=(1024, 4096)):
    import bit_quantized_gemm_repack_amd as hq
    import datagen

    N = K = 8192
    pts = []
    for M in Ms:
        d = datagen.dense_w4a16(M, N, K, act="f16", zp="fixed", key=(3,))
        plan = hq.Plan(N, K, hq.w4a16("f16"), max_m=M)
        w, meta = plan.repack(torch.from_numpy(d["codes"]).to(dev), d["scales"].to(dev))
        R = 32  # 32 weight copies of 33.6 MB: > 1 GB
        ws_ = [(w.clone(), meta.clone()) for _ in range(R)]
        a_ = [d["a"].to(dev) for _ in range(4)]
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws = plan.workspace(M, dev)
        byt = N * K // 2 + 2 * N * (K // 128) + 2 * M * K + 2 * M * N
        def check(out=out, d=d, M=M):
            from oracle import gemm as og

            rows = np.sort(np.random.default_rng(M).choice(M, 8, replace=False))
            ref = og.gemm_w4a16(d["a"][rows].double().numpy(), d["codes"], d["scales"].double().numpy(), 8,
                                out_fmt="f16")
            return og.check(out[rows].double().cpu().numpy(), ref["c64"], ref["tau"], "f16")

        pts.append(dict(name=f"M={M} N={N} K={K}", R=R, bytes=byt, flops=2 * M * N * K, peak=FP16_PEAK_TFLOPS,
                        mfma="f16", plan=plan.describe(M), check=check,
                        calls=lambda r, plan=plan, ws_=ws_, a_=a_, out=out, ws=ws:
                        [lambda: plan.gemm(a_[r % 4], ws_[r][0], ws_[r][1], out=out, ws=ws)]))
    return pts, "quantized GEMM TFLOPS vs M (dense W4A16 prefill)", \
        "dense W4A16 prefill: M in {1024,4096}, N = K = 8192, fp16 activations, uint4 weights (group 128, fp16 " \
        "scales, zero point 8), fp16 output", "f16"


def _w4a8_points(dev, Ms=(1, 16, 128, 1024), kinds=("mxfp4", "int")):
    import bit_quantized_gemm_repack_amd as hq
    import datagen

    N, K = 4096, 7168
    pts = []
    for kind in kinds:
        for M in Ms:
            d = datagen.w4a8_mxfp4(M, N, K) if kind == "mxfp4" else datagen.w4a8_int(M, N, K)
            plan = hq.Plan(N, K, hq.w4a8_mxfp4() if kind == "mxfp4" else hq.w4a8_int(), max_m=M)
            if kind == "mxfp4":
                w, meta = plan.repack(torch.from_numpy(d["codes"]).to(dev), e8m0=torch.from_numpy(d["e8m0"]).to(dev))
            else:
                w, meta = plan.repack(torch.from_numpy(d["codes"]).to(dev), d["scales"].to(dev))
            R = 64  # 64 copies of ~15.6 MB: > 1 GB
            ws_ = [(w.clone(), meta.clone()) for _ in range(R)]
            a, sa = d["a_codes"].to(dev), d["a_scale"].to(dev)
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = plan.workspace(M, dev)
            meta_b = N * K // 32 if kind == "mxfp4" else 2 * N * (K // 128)
            byt = N * K // 2 + meta_b + M * K + 4 * M + 2 * M * N
            def check(out=out, d=d, M=M, kind=kind):
                from oracle import gemm as og

                rows = np.sort(np.random.default_rng(M).choice(M, min(M, 8), replace=False))
                ac, asc = d["a_codes"].numpy()[rows], d["a_scale"].numpy()[rows]
                if kind == "mxfp4":
                    ref = og.gemm_mxfp4_fp8(ac, asc, d["codes"], d["e8m0"])
                else:
                    ref = og.gemm_int4_int8(ac, asc, d["codes"], d["scales"].double().numpy())
                return og.check(out[rows].double().cpu().numpy(), ref["c64"], ref["tau"], "bf16")

            pts.append(dict(name=f"{kind} M={M} N={N} K={K}", R=R, bytes=byt, flops=2 * M * N * K,
                            peak=FP8_PEAK_TFLOPS, mfma="fp8_fp4" if kind == "mxfp4" else "int8", plan=plan.describe(M),
                            check=check, calls=lambda r, plan=plan, ws_=ws_, a=a, sa=sa, out=out, ws=ws:
                            [lambda: plan.gemm(a, ws_[r][0], ws_[r][1], a_scale=sa, out=out, ws=ws)]))
        del d
    return pts, "quantized GEMM TFLOPS and effective HBM GB/s vs M (W4A8)", \
        "dense W4A8: M in {1,16,128,1024}, N = 4096, K = 7168; MXFP4 weights (E8M0 scales) x fp8 e4m3 " \
        "activations, and INT4 weights (fp16 scales, zero point 8) x int8 activations; bf16 output", "f8/i8"


def _w8a16_points(dev):
    import bit_quantized_gemm_repack_amd as hq
    import datagen

    N = K = 4096
    pts = []
    for M in (1, 16, 64, 1024):
        d = datagen.dense_w8a16(M, N, K, act="bf16")
        plan = hq.Plan(N, K, hq.w8a16("bf16"), max_m=M)
        w, meta = plan.repack(torch.from_numpy(d["codes"]).to(dev), d["scales"].to(dev))
        R = 64  # 64 copies of 17 MB: > 1 GB
        ws_ = [(w.clone(), meta.clone()) for _ in range(R)]
        a = d["a"].to(dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = plan.workspace(M, dev)
        byt = N * K + 2 * N * (K // 128) + 2 * M * K + 2 * M * N
        pts.append(dict(name=f"M={M} N={N} K={K}", R=R, bytes=byt, flops=2 * M * N * K, peak=FP16_PEAK_TFLOPS,
                        plan=plan.describe(M),
                        calls=lambda r, plan=plan, ws_=ws_, a=a, out=out, ws=ws:
                        [lambda: plan.gemm(a, ws_[r][0], ws_[r][1], out=out, ws=ws)]))
    return pts, "quantized GEMM TFLOPS and effective HBM GB/s vs M (W8A16)", \
        "dense W8A16: M in {1,16,64,1024}, N = K = 4096, bf16 activations, INT8 weights (group 128, bf16 scales, " \
        "zero point 128), bf16 output", "bf16"


def _w2a16_points(dev, bits=2):
    import bit_quantized_gemm_repack_amd as hq
    import datagen

    N = K = 4096
    gen, desc, zp = {2: (datagen.dense_w2a16, hq.w2a16, 2), 3: (datagen.dense_w3a16, hq.w3a16, 4)}[bits]
    pts = []
    for M in (1, 16, 64, 1024):
        d = gen(M, N, K, act="bf16")
        plan = hq.Plan(N, K, desc("bf16"), max_m=M)
        w, meta = plan.repack(torch.from_numpy(d["codes"]).to(dev), d["scales"].to(dev))
        R = 200  # 200 copies of >= 5 MB: > 1 GB
        ws_ = [(w.clone(), meta.clone()) for _ in range(R)]
        a = d["a"].to(dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = plan.workspace(M, dev)
        byt = N * K * bits // 8 + 2 * N * (K // 128) + 2 * M * K + 2 * M * N
        pts.append(dict(name=f"M={M} N={N} K={K}", R=R, bytes=byt, flops=2 * M * N * K, peak=FP16_PEAK_TFLOPS,
                        plan=plan.describe(M),
                        calls=lambda r, plan=plan, ws_=ws_, a=a, out=out, ws=ws:
                        [lambda: plan.gemm(a, ws_[r][0], ws_[r][1], out=out, ws=ws)]))
    return pts, f"quantized GEMM TFLOPS and effective HBM GB/s vs M (W{bits}A16)", \
        f"dense W{bits}A16: M in {{1,16,64,1024}}, N = K = 4096, bf16 activations, INT{bits} weights (group 128, " \
        f"bf16 scales, zero point {zp}), bf16 output", "bf16"


def _mxint4_points(dev, nv=False):
    import bit_quantized_gemm_repack_amd as hq
    import datagen

    N = K = 4096
    pts = []
    for M in (1, 16, 64, 1024):
        if nv:
            d = datagen.w4a16_nvfp4(M, N, K, act="bf16")
            plan = hq.Plan(N, K, hq.w4a16_nvfp4("bf16"), max_m=M)
            w, meta = plan.repack(torch.from_numpy(d["codes"]).to(dev), torch.from_numpy(d["tscale"]).to(dev),
                                  e8m0=torch.from_numpy(d["e4m3"]).to(dev))
        else:
            d = datagen.w4a16_mxint4(M, N, K, act="bf16")
            plan = hq.Plan(N, K, hq.w4a16_mxint4("bf16"), max_m=M)
            w, meta = plan.repack(torch.from_numpy(d["codes"]).to(dev), e8m0=torch.from_numpy(d["e8m0"]).to(dev))
        R = 128  # 128 copies of 8.9 MB: > 1 GB
        ws_ = [(w.clone(), meta.clone()) for _ in range(R)]
        a = d["a"].to(dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = plan.workspace(M, dev)
        byt = N * K // 2 + N * (K // (16 if nv else 32)) + 2 * M * K + 2 * M * N
        pts.append(dict(name=f"M={M} N={N} K={K}", R=R, bytes=byt, flops=2 * M * N * K, peak=FP16_PEAK_TFLOPS,
                        plan=plan.describe(M),
                        calls=lambda r, plan=plan, ws_=ws_, a=a, out=out, ws=ws:
                        [lambda: plan.gemm(a, ws_[r][0], ws_[r][1], out=out, ws=ws)]))
    if nv:
        return pts, "quantized GEMM TFLOPS and effective HBM GB/s vs M (W4A16-NVFP4)", \
            "dense W4A16-NVFP4: M in {1,16,64,1024}, N = K = 4096, bf16 activations, NVFP4 weights (one E4M3 scale " \
            "per 16 k, fp32 tensor scale), bf16 output", "bf16"
    return pts, "quantized GEMM TFLOPS and effective HBM GB/s vs M (W4A16-MXINT4)", \
        "dense W4A16-MXINT4: M in {1,16,64,1024}, N = K = 4096, bf16 activations, MXINT4 weights (one E8M0 scale " \
        "per 32 k), bf16 output", "bf16"


def _w4a4_points(dev):
    import bit_quantized_gemm_repack_amd as hq
    import datagen

    N, K = 4096, 7168
    pts = []
    for M in (1, 16, 128, 1024):
        d = datagen.w4a4_mxfp4(M, N, K)
        plan = hq.Plan(N, K, hq.w4a4_mxfp4(), max_m=M)
        w, meta = plan.repack(torch.from_numpy(d["codes"]).to(dev), e8m0=torch.from_numpy(d["e8m0"]).to(dev))
        R = 64  # 64 copies of 15.6 MB: > 1 GB
        ws_ = [(w.clone(), meta.clone()) for _ in range(R)]
        a = torch.from_numpy(d["a_codes"]).to(dev)
        ea = hq.mx_scales_group_major(torch.from_numpy(d["a_e8m0"])).to(dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = plan.workspace(M, dev)
        byt = N * K // 2 + N * K // 32 + M * K // 2 + M * K // 32 + 2 * M * N
        pts.append(dict(name=f"M={M} N={N} K={K}", R=R, bytes=byt, flops=2 * M * N * K, peak=FP4_PEAK_TFLOPS,
                        plan=plan.describe(M),
                        calls=lambda r, plan=plan, ws_=ws_, a=a, ea=ea, out=out, ws=ws:
                        [lambda: plan.gemm(a, ws_[r][0], ws_[r][1], a_scale=ea, out=out, ws=ws)]))
    return pts, "quantized GEMM TFLOPS and effective HBM GB/s vs M (W4A4)", \
        "dense W4A4: M in {1,16,128,1024}, N = 4096, K = 7168; MXFP4 activations x MXFP4 weights (E2M1 codes, " \
        "E8M0 scales per 32), bf16 output", "f4"


def _moe_points(dev, Ts=(1, 4, 8, 32, 512, 4096), acts=("bf16", "fp8"), slot_Ts=(1, 4, 8, 32)):
    import bit_quantized_gemm_repack_amd as hq
    import datagen

    E, H, I, topk = 256, 7168, 256, 8
    wts = datagen.moe_weights(E, H, I, key=(5,))
    per_expert = 2 * I * H // 2 + 2 * (2 * I) * (H // 128) + H * I // 2 + 2 * H * (I // 128)
    pts = []
    for act in acts:
        q = hq.w4a16("bf16", scale="f16") if act == "bf16" else hq.w4a8_fp8(scale="f16")
        p1 = hq.MoePlan(2 * I, H, q, E, 4096, "silu_mul" if act == "bf16" else "silu_mul_qfp8")
        p2 = hq.MoePlan(H, I, q, E, 4096, "topk_combine")
        w1, m1 = p1.repack(torch.from_numpy(wts["w1"]).to(dev), wts["s1"].to(dev))
        w2, m2 = p2.repack(torch.from_numpy(wts["w2"]).to(dev), wts["s2"].to(dev))
        C = 2  # two copies of the 727 MB expert weights: > 1 GB
        cp = [(w1, m1, w2, m2)] + [(w1.clone(), m1.clone(), w2.clone(), m2.clone()) for _ in range(C - 1)]
        abytes = 2 if act == "bf16" else 1

        def routings(T):
            # A pass touches only its routed experts' weights: at small T
            # those of one routing would stay in the 256 MB last-level cache
            # from pass to pass, so the passes cycle through several routings
            # (and both weight copies) until a graph touches >= 600 MB.
            first = datagen.moe_routing(T)
            hit0 = int(np.unique(first["topk_ids"]).size)
            n = int(min(16, max(1, -(-600e6 // (C * hit0 * per_expert)))))
            rts = [first] + [datagen.moe_routing(T, key=(5, j)) for j in range(1, n)]
            hit = float(np.mean([np.unique(rt["topk_ids"]).size for rt in rts]))
            ids = [torch.from_numpy(rt["topk_ids"]).to(dev) for rt in rts]
            tw = [torch.from_numpy(rt["topk_w"]).to(dev) for rt in rts]
            return n, hit, ids, tw

        for T in Ts:
            n_rt, hit, ids, tw = routings(T)
            x = datagen.moe_activations(T, act=act)
            xa = (x["x"] if act == "bf16" else x["x_codes"]).to(dev)
            xs = None if act == "bf16" else x["x_scale"].to(dev)
            bm = p1.block_m(T, topk)
            mp = hq.moe_max_padded(T, topk, E, bm)
            sid = torch.empty(mp, dtype=torch.int32, device=dev)
            bex = torch.empty(max(mp // bm, 1), dtype=torch.int32, device=dev)
            npad = torch.empty(1, dtype=torch.int32, device=dev)
            inter = torch.empty((mp, I), dtype=torch.bfloat16 if act == "bf16" else torch.uint8, device=dev)
            iscale = None if act == "bf16" else torch.empty(mp, dtype=torch.float32, device=dev)
            y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            ws1, ws2 = p1.moe_workspace(T, topk, dev), p2.moe_workspace(T, topk, dev)
            # weights of the experts hit (mean over the routings), A once (+
            # scale), the intermediate written once and read once, y once
            byt = int(hit * per_expert) + T * H * abytes + (4 * T if act == "fp8" else 0) + \
                2 * T * topk * I * abytes + 2 * T * H
            flops = 2 * T * topk * (2 * I * H + H * I)

            def calls(r, cp=cp, ids=ids, tw=tw, xa=xa, xs=xs, bm=bm, sid=sid, bex=bex, npad=npad, inter=inter,
                      iscale=iscale, y=y, ws1=ws1, ws2=ws2, T=T, p1=p1, p2=p2):
                w1_, m1_, w2_, m2_ = cp[r % C]
                ids_, tw_ = ids[r // C], tw[r // C]
                L = hq.lib()

                def align():
                    hq._check(L.hq_moe_align(T, topk, E, bm, hq._ptr(ids_), hq._ptr(sid), hq._ptr(bex),
                                             hq._ptr(npad), hq._stream_ptr(ids_.device)))

                def gate_up():
                    p1.moe_gemm(xa, T, topk, sid, bex, npad, w1_, m1_, a_scale=xs, out=inter, out_scale=iscale,
                                ws=ws1)

                def down():
                    p2.moe_gemm(inter, T, topk, sid, bex, npad, w2_, m2_, a_scale=iscale, topk_w=tw_, out=y, ws=ws2)

                return [align, gate_up, down]

            pts.append(dict(name=f"{act} T={T} (experts hit {hit:.0f}, {n_rt} routings)", R=C * n_rt, bytes=byt,
                            flops=flops, peak=FP16_PEAK_TFLOPS if act == "bf16" else FP8_PEAK_TFLOPS,
                            mfma="bf16" if act == "bf16" else "fp8",
                            plan=f"gate_up: {p1.describe(T, topk)} | down: {p2.describe(T, topk)}", calls=calls))
        for T in slot_Ts:
            # the unaligned path: rows indexed by routed slot, no align launch
            n_rt, hit, ids, tw = routings(T)
            x = datagen.moe_activations(T, act=act)
            xa = (x["x"] if act == "bf16" else x["x_codes"]).to(dev)
            xs = None if act == "bf16" else x["x_scale"].to(dev)
            S = T * topk
            inter = torch.empty((S, I), dtype=torch.bfloat16 if act == "bf16" else torch.uint8, device=dev)
            iscale = None if act == "bf16" else torch.empty(S, dtype=torch.float32, device=dev)
            y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            ws1 = p1.moe_workspace(T, topk, dev) if act == "fp8" else None
            # the experts hit once each (an expert picked by two slots is read
            # twice, from the cache the second time: not counted), A, the slot
            # rows written and read, y
            byt = int(hit * per_expert) + T * H * abytes + (4 * T if act == "fp8" else 0) + \
                2 * S * I * abytes + 2 * T * H
            flops = 2 * S * (2 * I * H + H * I)

            def calls(r, cp=cp, ids=ids, tw=tw, xa=xa, xs=xs, inter=inter, iscale=iscale, y=y, ws1=ws1, T=T,
                      p1=p1, p2=p2):
                w1_, m1_, w2_, m2_ = cp[r % C]
                ids_, tw_ = ids[r // C], tw[r // C]

                def gate_up():
                    p1.moe_gemm_by_slot(xa, T, topk, ids_, w1_, m1_, a_scale=xs, out=inter, out_scale=iscale,
                                        ws=ws1)

                def down():
                    p2.moe_gemm_by_slot(inter, T, topk, ids_, w2_, m2_, a_scale=iscale, topk_w=tw_, out=y)

                return [gate_up, down]

            pts.append(dict(name=f"{act} T={T} by slot (experts hit {hit:.0f}, {n_rt} routings)", R=C * n_rt,
                            bytes=byt, flops=flops, peak=FP16_PEAK_TFLOPS if act == "bf16" else FP8_PEAK_TFLOPS,
                            mfma="bf16" if act == "bf16" else "fp8",
                            plan="gate_up + down by slot (skinny kernel, slot and token modes)", calls=calls))
    return pts, "MoE layer TFLOPS and effective HBM GB/s vs T", \
        "MoE layer on one GPU's tensor-parallel share: 256 experts, top-8, hidden 7168, intermediate 256; " \
        "align + gate_up (SiLU * up; bf16, or fp8 requant for W4A8-FP8) + down with the top-k combine; INT4 " \
        "weights (group 128, fp16 scales, zero point 8); T in {1,4,8,32,512,4096}; the unaligned by-slot path " \
        "(gate_up + down, no align) at T in {1,4,8,32}; small T cycles through routings so passes stay cold", \
        "bf16/f8"


def graph_time_point(p, steps, warmup):
    """Mean time of one pass of the point's calls, in ms: one HIP graph holds a
    pass over every weight copy of the rotating pool (R passes back to back,
    so the weights of consecutive passes are cold in the last-level cache),
    replayed between two events on the replay stream; the launch gaps inside
    the graph are included, the host's per-graph launch is amortised over R."""
    R = p["R"]
    for r in range(min(R, 2)):
        for c in p["calls"](r):
            c()
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for c in p["calls"](0):
            c()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(R):
            for c in p["calls"](r):
                c()
    g.replay()  # the first launch uploads the graph
    for _ in range(max(1, -(-warmup // R))):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-steps // R))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * R)


def eager_call_times(p, steps, hip, L):
    """Median device duration of each of the point's calls (dispatch-bracketing
    events, eager launches), in us: the split of a multi-call point."""
    import bit_quantized_gemm_repack_amd as hq

    n = len(p["calls"](0))
    times = [[] for _ in range(n)]
    for i in range(steps):
        pend = []
        for j, c in enumerate(p["calls"](i % p["R"])):
            a, b = hip.event(), hip.event()
            hq._check(L.hq_time_next_launch(a, b))
            c()
            pend.append((j, a, b))
        torch.cuda.synchronize()
        for j, a, b in pend:
            times[j].append(hip.elapsed_ms(a, b) * 1e3)
            hip.destroy(a)
            hip.destroy(b)
    return [round(float(np.median(t)), 3) for t in times]


def point_result(p, ms, ceil=None):
    """Per-point figures from its graph-replay time `ms`."""
    us = ms * 1e3
    t_hbm = p["bytes"] / (HBM_PEAK_GBS * 1e3)
    t_mfma = p["flops"] / (p["peak"] * 1e6)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    r = {"point": p["name"], "us": round(us, 3), "GBps": round(p["bytes"] / us / 1e3, 1),
         "TFLOPS": round(p["flops"] / us / 1e6, 2), "bound": bound, "roofline_frac": round(max(t_hbm, t_mfma) / us, 4),
         "mfma_frac": round(t_mfma / us, 4), "hbm_frac": round(t_hbm / us, 4), "bytes": p["bytes"],
         "flops": p["flops"], "plan": p["plan"]}
    kind = p.get("mfma") or {FP16_PEAK_TFLOPS: "bf16", FP8_PEAK_TFLOPS: "fp8", FP4_PEAK_TFLOPS: "fp4"}[p["peak"]]
    r["mfma_type"] = kind
    if ceil:
        r["frac_of_measured_mfma"] = round(r["TFLOPS"] / ceil[kind], 4)
    if bound == "mfma":
        r["roofline"] = {"bound": "mfma", "achieved": r["TFLOPS"], "peak": p["peak"], "unit": "TFLOP/s",
                         "frac": r["mfma_frac"], "traffic": None}
    else:
        r["roofline"] = {"bound": "hbm", "achieved": r["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": r["hbm_frac"], "traffic": None}
    if p.get("check"):
        ok, lit, ratio = p["check"]()
        if not ok.all():
            raise SystemExit(f"bench: output check of {p['name']} failed ({int((~ok).sum())} outputs, "
                             f"max err/tau {ratio.max():.3g})")
        r["spot_check"] = {"rows": int(ok.shape[0]), "max_err_over_tau": round(float(ratio.max()), 4),
                           "literal_tau_pass_frac": round(float(lit.mean()), 6)}
    return r


def run_points_workload(args, builder):
    import bit_quantized_gemm_repack_amd as hq

    dev = torch.device("cuda:0")
    hip = Hip()
    L = hq.lib()
    print(f"[bench] preparing the {args.workload} workload", file=sys.stderr, flush=True)
    pts, metric, workload, dtype = builder(dev)
    ceil = mfma_ceilings(hip, L, dev)
    points, step_ms = [], 0.0
    with GpuStateSampler() as smp:
        for p in pts:
            ms = graph_time_point(p, args.steps, args.warmup)
            step_ms += ms
            r = point_result(p, ms, ceil)
            if len(p["calls"](0)) > 1:
                r["calls_us_eager"] = eager_call_times(p, min(args.steps, 20), hip, L)
            points.append(r)
            print(f"[bench] {p['name']}: {r['us']:.1f} us ({r['bound']} {r['roofline_frac']:.3f})", file=sys.stderr,
                  flush=True)
    step_bytes = sum(p["bytes"] for p in pts)
    step_flops = sum(p["flops"] for p in pts)
    dom = int(np.argmax([q["us"] for q in points]))
    roof = dict(points[dom]["roofline"], point=points[dom]["point"], us=points[dom]["us"])
    if roof["bound"] == "mfma":
        roof["measured_peak"] = ceil[points[dom]["mfma_type"]]
        roof["frac_of_measured_peak"] = points[dom]["frac_of_measured_mfma"]
    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = _cpu_sample(args.workload, args.cpu_budget)
    line = {"metric": metric, "value": round(step_flops / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "config": {"workload": workload, "points_per_step": len(pts), "step_bytes": step_bytes,
                       "step_flops": step_flops, "gbps_per_step_time": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
                       "timing": "per point: one HIP graph of its calls over every weight copy of the pool, "
                                 "events around the replays; the step is the sum over the points"},
            "roofline": roof, "cpu_baseline": cpu, "mfma_ceilings_TFLOPS": ceil, "gpu_state": smp.summary(),
            "points": points}
    print(json.dumps(line), flush=True)


# The MFMA-bound and MoE targets measured beside the decode line (bench.py
# with no --workload): each entry is one point of another workload, timed by
# graph replay like the decode step, with its roofline, an output check on
# sampled rows where the oracle is cheap, and a bounded CPU-oracle sample.
EXTRA = (("prefill_f16_M4096", "prefill", lambda dev: _prefill_points(dev, Ms=(4096,))),
         ("w4a8_mxfp4_fp8_M1024", "w4a8", lambda dev: _w4a8_points(dev, Ms=(1024,), kinds=("mxfp4",))),
         ("w4a8_int4_int8_M1024", "w4a8int", lambda dev: _w4a8_points(dev, Ms=(1024,), kinds=("int",))),
         ("moe_bf16_T4096", "moe", lambda dev: _moe_points(dev, Ts=(4096,), acts=("bf16",), slot_Ts=())),
         ("moe_fp8_T4096", "moe", lambda dev: _moe_points(dev, Ts=(4096,), acts=("fp8",), slot_Ts=())),
         ("moe_bf16_T1_by_slot", "moe", lambda dev: _moe_points(dev, Ts=(), acts=("bf16",), slot_Ts=(1,))))


def measure_extra(args, dev, hip, L, cpu_budget):
    ceil = mfma_ceilings(hip, L, dev)
    out = {"mfma_ceilings_TFLOPS": ceil}
    for name, cpu_kind, builder in EXTRA:
        print(f"[bench] extra: {name}", file=sys.stderr, flush=True)
        pts, _, workload, dtype = builder(dev)
        p = pts[0]
        steps = max(10, min(args.steps, 50))
        r = point_result(p, graph_time_point(p, steps, min(args.warmup, 5)), ceil)
        if len(p["calls"](0)) > 1:
            r["calls_us_eager"] = eager_call_times(p, 10, hip, L)
        r["workload"] = workload
        r["dtype"] = dtype
        r["steps"] = steps
        if cpu_budget > 0:
            r["cpu_baseline"] = _cpu_sample(cpu_kind, cpu_budget)
        out[name] = r
        print(f"[bench] extra {name}: {r['us']:.1f} us ({r['bound']} {r['roofline_frac']:.3f})", file=sys.stderr,
              flush=True)
        del pts, p
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def _cpu_sample(workload, budget):
    """The oracle on a row sample of the workload, in TFLOP/s of oracle work."""
    import datagen
    from oracle import gemm as og

    flops, secs, runs = 0, 0.0, 0
    while secs < budget:
        if workload == "prefill":
            M, N, K = 8, 8192, 8192
            d = datagen.dense_w4a16(M, N, K, act="f16", zp="fixed", key=(3,))
            t0 = time.perf_counter()
            og.gemm_w4a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), 8, out_fmt="f16")
            what = "dense W4A16 M=8 rows of N = K = 8192"
        elif workload == "w8a16":
            M, N, K = 8, 4096, 4096
            d = datagen.dense_w8a16(M, N, K, act="bf16")
            t0 = time.perf_counter()
            og.gemm_w8a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), 128, out_fmt="bf16")
            what = "dense W8A16 M=8 N=K=4096"
        elif workload == "w2a16":
            M, N, K = 8, 4096, 4096
            d = datagen.dense_w2a16(M, N, K, act="bf16")
            t0 = time.perf_counter()
            og.gemm_w2a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), 2, out_fmt="bf16")
            what = "dense W2A16 M=8 N=K=4096"
        elif workload == "w3a16":
            M, N, K = 8, 4096, 4096
            d = datagen.dense_w3a16(M, N, K, act="bf16")
            t0 = time.perf_counter()
            og.gemm_w3a16(d["a"].double().numpy(), d["codes"], d["scales"].double().numpy(), 4, out_fmt="bf16")
            what = "dense W3A16 M=8 N=K=4096"
        elif workload == "mxint4":
            M, N, K = 8, 4096, 4096
            d = datagen.w4a16_mxint4(M, N, K, act="bf16")
            t0 = time.perf_counter()
            og.gemm_mxint4_w16(d["a"].double().numpy(), d["codes"], d["e8m0"], out_fmt="bf16")
            what = "dense W4A16-MXINT4 M=8 N=K=4096"
        elif workload == "nvfp4":
            M, N, K = 8, 4096, 4096
            d = datagen.w4a16_nvfp4(M, N, K, act="bf16")
            t0 = time.perf_counter()
            og.gemm_nvfp4_w16(d["a"].double().numpy(), d["codes"], d["e4m3"], float(d["tscale"][0]), out_fmt="bf16")
            what = "dense W4A16-NVFP4 M=8 N=K=4096"
        elif workload == "w4a4":
            M, N, K = 16, 4096, 7168
            d = datagen.w4a4_mxfp4(M, N, K)
            t0 = time.perf_counter()
            og.gemm_mxfp4_mxfp4(d["a_codes"], d["a_e8m0"], d["codes"], d["e8m0"])
            what = "W4A4-MXFP4 M=16 N=4096 K=7168"
        elif workload == "w4a8":
            M, N, K = 16, 4096, 7168
            d = datagen.w4a8_mxfp4(M, N, K)
            t0 = time.perf_counter()
            og.gemm_mxfp4_fp8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["e8m0"])
            what = "W4A8-MXFP4 M=16 N=4096 K=7168"
        elif workload == "w4a8int":
            M, N, K = 16, 4096, 7168
            d = datagen.w4a8_int(M, N, K)
            t0 = time.perf_counter()
            og.gemm_int4_int8(d["a_codes"].numpy(), d["a_scale"].numpy(), d["codes"], d["scales"].double().numpy())
            what = "W4A8-INT4xINT8 M=16 N=4096 K=7168"
        else:
            from oracle import moe as om

            M, N, K = 8, 512, 7168  # one token's 8 gate_up rows, each through its own expert
            rt = datagen.moe_routing(1)
            wts = datagen.moe_weights(256, 7168, 256, key=(5,), experts=rt["topk_ids"][0])
            x = datagen.moe_activations(1)["x"].double().numpy()
            rows = np.repeat(x, 8, axis=0)
            t0 = time.perf_counter()
            om.gate_up(rows, rt["topk_ids"][0], wts["w1"], wts["s1"].double().numpy(), 256)
            what = "MoE gate_up of one token (8 experts, N = 512, K = 7168)"
        secs += time.perf_counter() - t0
        flops += 2 * M * N * K
        runs += 1
    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{runs} oracle runs of {what} (unpack + float64 dequantise + float64 GEMM), {secs:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotations", type=int, default=4)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="decode: skip the prefill / W4A8 / MoE points reported in 'extra'")
    ap.add_argument("--autotune", action="store_true",
                    help="decode: install a measured execution choice per point (hq_plan_autotune) first")
    ap.add_argument("--workload", choices=("decode", "quant", "prefill", "w4a8", "w4a4", "w8a16", "w2a16", "w3a16", "mxint4", "nvfp4", "moe"),
                    default="decode",
                    help="decode: the dense W4A16 decode sweep (default); quant: the per-token quantiser; "
                         "prefill / w4a8 / w4a4 / w8a16 / w2a16 / w3a16 / mxint4 / nvfp4 / moe: the other GEMM workloads")
    ap.add_argument("--write-profiles", metavar="RUN_DIR",
                    help="CPU only: write the profiles/ summaries from rocprofv3 outputs in RUN_DIR and exit")
    args = ap.parse_args()
    if args.write_profiles:
        write_profiles(args.write_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested); the sharded "
              "form is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    if args.workload == "quant":
        run_quant(args)
        return
    if args.workload in ("prefill", "w4a8", "w4a4", "w8a16", "w2a16", "w3a16", "mxint4", "nvfp4", "moe"):
        run_points_workload(args, {"prefill": _prefill_points, "w4a8": _w4a8_points, "w4a4": _w4a4_points,
                                   "w8a16": _w8a16_points, "w2a16": _w2a16_points,
                                   "w3a16": lambda dev: _w2a16_points(dev, 3), "mxint4": _mxint4_points,
                                   "nvfp4": lambda dev: _mxint4_points(dev, nv=True),
                                   "moe": _moe_points}[args.workload])
        return

    import bit_quantized_gemm_repack_amd as hq

    dev = torch.device("cuda:0")
    hip = Hip()
    L = hq.lib()
    print(f"[bench] preparing {len(SWEEP_M) * len(SWEEP_NK)} points x {args.rotations} rotations", file=sys.stderr,
          flush=True)
    points, shapes = make_points(dev, args.rotations, args.autotune)
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
    for g in graphs:  # a graph's first launch uploads it: once each, before the warm-up steps
        g.replay()
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with GpuStateSampler() as smp:
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

    # --- per-call durations, eager (dispatch-bracketing events) -------------
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
    for j, p in enumerate(points):
        ms = [hip.elapsed_ms(*evs[i * n + j]) for i in range(args.steps)]
        us = float(np.mean(ms)) * 1e3
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
    ceilings = measure_ceilings(points, hip, L, R, args.steps)
    for pp, us in zip(per_point, ceilings.pop("point_read_us")):
        pp["plain_read_of_weights_us"] = us

    # the roofline of the step: algorithmic bytes of the twelve calls over the
    # graph-replayed step time (events around the timed replays on the replay
    # stream), i.e. the mean call of the step with its launch gap included
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    mean_call_us = ms_per_step * 1e3 / n
    roof = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4), "traffic": measured_traffic([p["plan"] for p in per_point]),
            "kernel": "hq_gemm calls of the sweep: hq::qgemm_skinny / hq::qgemm_tiled",
            "mean_call_us": round(mean_call_us, 3), "mean_algorithmic_bytes": int(step_bytes / n),
            "timing": "graph-replayed step: events around the timed replays; mean call = step / 12"}

    cpu = None
    extra = None
    if not args.no_cpu:
        # the CPU oracle leg: every point's timed output against the oracle, then its timing
        max_ratio, lit_frac, n_out = check_points(points, shapes)
        print(f"[bench] output check against the oracle ok ({n_out} outputs, max err/tau {max_ratio:.3g}, "
              f"literal-tau pass fraction {lit_frac:.4f}); timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.cpu_budget)
        cpu["check"] = {"outputs": n_out, "max_err_over_tau": round(max_ratio, 4),
                        "literal_tau_pass_frac": round(lit_frac, 6)}
    del points, shapes, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_extra:
        extra = measure_extra(args, dev, hip, L, 0 if args.no_cpu else 2.5)

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
                   "weight_pool_rotations": R, "execution_choice": "autotuned" if args.autotune else "heuristic",
                   "timing": "HIP graph replay per step; per-call durations in 'points' from dispatch-bracketing "
                             "HIP events on eager launches"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "ceilings": dict(ceilings, frac_of_same_bytes_read=round(value / ceilings["same_bytes_read_GBps"], 4)),
        "gpu_state": smp.summary(),
        "points": per_point,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
