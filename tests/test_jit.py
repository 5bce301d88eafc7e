"""Run-time specialisation (hq_plan_set_jit, hq_jit_cache_key, hq_jit_prepare)
on the host: the cache key, the hipRTC compile into the code-object cache and
the cache file, without a device.  Launches are in tests/test_jit_gpu.py."""
import os
import re
import shutil
import subprocess
import sys

import pytest

import bit_quantized_gemm_repack_amd as hq

KEY = re.compile(r"^hq-(skinny|tiled)-gfx9[0-9a-f]+-[0-9a-f]{16}$")
PKG = os.path.dirname(hq.__file__)


def _decode_plan(**kw):
    return hq.Plan(4096, 4096, hq.w4a16("bf16", zp="u4"), max_m=64, **kw)


def test_key_form_and_determinism():
    p, q = _decode_plan(), _decode_plan()
    for m in (1, 4, 16, 64):
        k = p.jit_cache_key(m)
        assert KEY.match(k) and len(k) <= 63, k
        assert k == q.jit_cache_key(m)               # same plan contents, same key
    assert p.jit_cache_key(1).startswith("hq-skinny-gfx950-")
    r = hq.Plan(8192, 8192, hq.w4a16("f16"), max_m=1024)
    assert r.jit_cache_key(1024).startswith("hq-tiled-gfx950-")


def test_key_changes_with_every_field():
    p = _decode_plan()
    keys = {p.jit_cache_key(m) for m in (1, 2, 3, 4, 16, 17, 64)}
    assert len(keys) == 7                             # the row count is a constant of the kernel
    assert p.jit_cache_key(16, "gfx942") != p.jit_cache_key(16)
    assert hq.Plan(4096, 8192, hq.w4a16("bf16", zp="u4"), max_m=64).jit_cache_key(16) != p.jit_cache_key(16)
    assert hq.Plan(8192, 4096, hq.w4a16("bf16", zp="u4"), max_m=64).jit_cache_key(16) != p.jit_cache_key(16)
    assert hq.Plan(4096, 4096, hq.w4a16("f16", zp="u4"), max_m=64).jit_cache_key(16) != p.jit_cache_key(16)
    before = p.jit_cache_key(16)
    p.set_tuning(16, dict(kernel=1, tile_m=16, tile_n=32, waves=4, split_k=2, stages=4))
    assert p.jit_cache_key(16) != before              # the execution choice is part of the key
    p.set_tuning(16, None)
    assert p.jit_cache_key(16) == before


def _key_from_copy(pkg_dir, m=16):
    # a fresh interpreter (no device touched) loading the library copy in pkg_dir
    code = ("import sys; sys.path.insert(0, %r); import bit_quantized_gemm_repack_amd as hq; "
            "hq.LIB_PATH = %r; p = hq.Plan(4096, 4096, hq.w4a16('bf16', zp='u4'), max_m=64); "
            "print(p.jit_cache_key(%d))") % (os.path.dirname(PKG), os.path.join(pkg_dir, "libhq.so"), m)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env)
    assert out.returncode == 0, out.stderr[-2000:]
    return out.stdout.strip().splitlines()[-1]


def test_key_follows_the_kernel_sources(tmp_path):
    import torch
    if torch.cuda.is_initialized():
        pytest.skip("starts a child interpreter: only from a process that has not touched the GPU")
    same, edited = tmp_path / "same", tmp_path / "edited"
    for d in (same, edited):
        (d / "csrc").mkdir(parents=True)
        shutil.copy(os.path.join(PKG, "libhq.so"), d / "libhq.so")
        for f in os.listdir(os.path.join(PKG, "csrc")):
            if f.endswith(".h"):
                shutil.copy(os.path.join(PKG, "csrc", f), d / "csrc" / f)
    with open(edited / "csrc" / "qgemm_skinny_kernel.h", "a") as f:
        f.write("\n// an edit\n")
    here = _decode_plan().jit_cache_key(16)
    assert _key_from_copy(str(same)) == here          # where the sources sit does not matter
    assert _key_from_copy(str(edited)) != here        # what they say does


def test_prepare_compiles_into_the_cache_without_a_device(tmp_path):
    p = _decode_plan()
    p.set_jit(False, str(tmp_path))                   # the cache directory; specialisation stays off
    s0 = hq.jit_stats()
    p.jit_prepare(4)
    s1 = hq.jit_stats()
    assert s1["compiles"] == s0["compiles"] + 1 and s1["compile_seconds"] > s0["compile_seconds"]
    path = tmp_path / (p.jit_cache_key(4) + ".co")
    data = path.read_bytes()
    assert data.startswith(b"HQJIT1\n")
    name, code = data[7:].split(b"\n", 1)
    assert name.startswith(b"_ZN2hq12qgemm_skinny") and code.startswith(b"\x7fELF")
    assert [f for f in os.listdir(tmp_path) if ".tmp." in f] == []   # no temporary left behind
    p.jit_prepare(4)                                  # found on disk: no second compile
    s2 = hq.jit_stats()
    assert s2["compiles"] == s1["compiles"] and s2["disk_hits"] == s1["disk_hits"] + 1
    path.write_bytes(b"HQJIT1\n")                     # a damaged file is compiled again and replaced
    p.jit_prepare(4)
    assert hq.jit_stats()["compiles"] == s1["compiles"] + 1
    assert path.read_bytes()[7:].split(b"\n", 1)[1].startswith(b"\x7fELF")


def test_prepare_tiled_kernel(tmp_path):
    q = hq.Plan(4096, 4096, hq.w4a8_mxfp4(), max_m=1024)
    q.set_jit(False, str(tmp_path))
    q.jit_prepare(1024)
    data = (tmp_path / (q.jit_cache_key(1024) + ".co")).read_bytes()
    assert data[7:].startswith(b"_ZN2hq11qgemm_tiled")


def test_jit_argument_checks(tmp_path):
    p = _decode_plan()
    with pytest.raises(hq.HQError):
        p.jit_cache_key(0)
    with pytest.raises(hq.HQError):
        p.jit_cache_key(65)
    L = hq.lib()
    small = hq.ctypes.create_string_buffer(8)
    assert L.hq_jit_cache_key(p._h, 16, b"gfx950", small, 8) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_plan_set_jit(p._h, 2, None) == hq.HQ_ERR_INVALID_ARG
    assert L.hq_plan_set_jit(p._h, 1, b"x" * 600) == hq.HQ_ERR_INVALID_ARG
    moe = hq.MoePlan(512, 7168, hq.w4a16("bf16"), 256, 64, "silu_mul")
    with pytest.raises(hq.HQError):
        moe.set_jit(True)
    assert L.hq_jit_prepare(moe._h, 1, b"gfx950") == hq.HQ_ERR_UNSUPPORTED
    p.set_jit(True, str(tmp_path))
    p.set_jit(False)


OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="needs the ROCm disassembler")
@pytest.mark.parametrize("quant,m", [("w4a8_mxfp4", 16), ("w4a8_mxfp4", 1024), ("w4a8_fp8", 16), ("w4a8_fp8", 1024),
                                     ("w4a4_mxfp4", 16)])
def test_jit_scaled_mfma_scales_in_vgprs(quant, m, tmp_path):
    # the scaled matrix instruction reads its E8M0 scales from VGPRs only; the
    # run-time compiler (whichever hipRTC the process loaded) must not be left
    # to place a constant scale in a scalar register
    p = hq.Plan(4096, 7168, getattr(hq, quant)(), max_m=m)
    p.set_jit(False, str(tmp_path))
    p.jit_prepare(m)
    code = (tmp_path / (p.jit_cache_key(m) + ".co")).read_bytes()[7:].split(b"\n", 1)[1]
    (tmp_path / "k.o").write_bytes(code)
    asm = subprocess.run([OBJDUMP, "-d", str(tmp_path / "k.o")], capture_output=True, text=True, timeout=120).stdout
    lines = [ln for ln in asm.splitlines() if "v_mfma_scale_f32_16x16x128_f8f6f4" in ln]
    assert lines, "no scaled matrix instruction in the kernel"
    bad = [ln for ln in lines if re.search(r",\s*s\d+", ln.split("//")[0]) or "Invalid" in ln]
    assert not bad, bad[:3]
