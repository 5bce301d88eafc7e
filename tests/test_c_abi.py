"""The C ABI from C: tests/c/hq_c_consumer.c, compiled as C99 with warnings as
errors against include/hq.h and linked to the built libhq.so, runs its plan,
size and rejection checks (no device work) and prints "ok"."""
import os
import shutil
import subprocess

import pytest

import bit_quantized_gemm_repack_amd as hq

HERE = os.path.dirname(__file__)
ROOT = os.path.dirname(HERE)
PKG = os.path.dirname(hq.__file__)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_c99_consumer(tmp_path):
    import torch
    if torch.cuda.is_initialized():
        pytest.skip("starts a child program: only from a process that has not touched the GPU")
    hq.lib()                                   # the library is built
    exe = str(tmp_path / "hq_c_consumer")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Wpedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c", "hq_c_consumer.c"), "-L", PKG, "-l:libhq.so", "-Wl,-rpath," + PKG, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stderr[-3000:]
