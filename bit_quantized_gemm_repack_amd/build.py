"""Build the HIP library (libhq.so) in-tree for gfx950 with hipcc.

Every source is compiled to an object in parallel, then linked into
``bit_quantized_gemm_repack_amd/libhq.so``.  HIP device code is built with
packed-FP32 instruction selection disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhq.so")
ARCH = os.environ.get("HQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = ["-O3", "-std=c++20", "-fPIC", "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]
DEVICE = [f"--offload-arch={ARCH}", "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Matrix-instruction results in ordinary VGPRs, so that the per-group
# epilogues read them without a v_accvgpr_read copy each; sources named
# *_f16.hip (an fp16 k loop without per-group epilogue) keep the default.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
# hipRTC for the run-time specialised kernels (hq_plan_set_jit)
LINK = ["-lhiprtc", "-Wl,-z,defs"]  # every symbol resolved at link time


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE + ([] if src.endswith("_f16.hip") else VGPR_FORM)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *DEVICE, "-shared", "-fPIC", "-o", tmp, *objs, *LINK]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
