"""CPU oracle for the quantized-GEMM hot path.  TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct statement of what the GPU
path computes: scalar unpack of the packed 4-bit codes, exact dequantisation
to float64, and a float64-accumulated matrix product.  It exists to check the
HIP kernels and is never part of the product path: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with ``bit_quantized_gemm_repack_amd`` (the
library); the only thing both sides consume is the seeded input generator in
``datagen``, which holds none of the method's arithmetic.

What the method computes comes from the Humming pages, which describe it only
in prose:

* Humming: open-source kernel library for quantized inference (news.ditty.ir),
  summary: every supported format is mapped onto one description in which the
  weight codes, the scales and the zero points are separate parameters; the
  supported combinations include WnA16, W4A8 and the MoE grouped path.
* Ant Group e vLLM lancam a biblioteca open source Humming (aube.news), body:
  INT4 stores one weight in 4 bits; the library covers dense and MoE layers.
* cocoloop.cn (vi/fr), section on the format list: MXFP4 is one of the
  supported weight formats, and W4A8 is run on FP8 activations.

The pages print no formula, layout, worked example or numeric result.  The
number formats follow the OCP Microscaling (MX) v1.0 specification (E2M1
elements, E8M0 shared scales, 32-element blocks) and the OCP 8-bit floating
point specification (E4M3).  Every reading taken where the pages are silent is
listed in the module docstrings and in the design notes of the repository.

Modules
-------
formats  code-value tables (E2M1, E8M0, E4M3), nibble unpack, exact
         round-to-nearest-even to fp16 / bf16 / e4m3.
gemm     dense W4A16, W4A8 (MXFP4 x FP8 and INT4 x INT8), W4A4 (MXFP4 x
         MXFP4) oracles and the per-output tolerance.
moe      the grouped MoE layer: align invariants, gate_up + SiLU*mul (+ fp8
         requant), down + top-k combine.
quant    the per-token (per-row) activation quantiser that feeds W4A8:
         s = max|x| / Q, codes = RNE(x / s) as fp8 e4m3 or int8; and the
         MXFP4 block quantiser (OCP MX v1.0) of W4A4 activations.

Parity status: every function is pinned by tests/test_oracle.py,
tests/test_quant_oracle.py and tests/test_moe_oracle.py against
hand-worked examples (tests/golden), code tables derived from the format
definitions, torch's fp8 decoders, exact rational brute force and
invariants.  No function is "parity unpinned".
"""
