"""Python binding of the MI355X quantized GEMM library (libhq.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/hq.h``.  PyTorch supplies the
device memory (tensors) and the stream (the current HIP stream); there is no
CPU fallback, and every entry point raises if the library is not built or a
tensor is not on the GPU.

Quick use::

    import bit_quantized_gemm_repack_amd as hq
    plan = hq.Plan(n=4096, k=4096, quant=hq.w4a16(act="bf16", zp="u4"), max_m=64)
    w, meta = plan.repack(codes, scales, zeros)        # canonical -> device layout
    out = plan.gemm(a, w, meta)                         # [m, n] bf16
"""
from __future__ import annotations

import ctypes
import json
import os
import re
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhq.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "hq.h")

# ------------------------------------------------------------------ enums --
HQ_OK, HQ_ERR_INVALID_ARG, HQ_ERR_UNSUPPORTED, HQ_ERR_WORKSPACE, HQ_ERR_HIP, HQ_ERR_INTERNAL = range(6)
F16, BF16, F32, FP8_E4M3, INT8, U4, FP4_E2M1, E8M0, I32, U8, U2, U3, I4 = range(13)
ZP_NONE, ZP_FIXED, ZP_PER_GROUP_U4 = range(3)
ASCALE_NONE, ASCALE_PER_TOKEN_F32, ASCALE_MX_E8M0 = range(3)
GEMM_DENSE, GEMM_GROUPED = range(2)
EPI_NONE, EPI_SILU_MUL, EPI_SILU_MUL_QFP8, EPI_TOPK_COMBINE, EPI_I32_ACC = range(5)
PEAK_F16, PEAK_BF16, PEAK_FP8, PEAK_FP8_FP4, PEAK_FP4, PEAK_INT8 = range(6)
MFMA_AUTO, MFMA_F16, MFMA_BF16, MFMA_FP8, MFMA_INT8, MFMA_FP8_FP4, MFMA_FP4 = range(7)
_MFMA = {None: MFMA_AUTO, "auto": MFMA_AUTO, "f16": MFMA_F16, "bf16": MFMA_BF16, "fp8": MFMA_FP8,
         "int8": MFMA_INT8, "fp8xfp4": MFMA_FP8_FP4, "fp4": MFMA_FP4}

_DT = {"f16": F16, "bf16": BF16, "fp8": FP8_E4M3, "int8": INT8}
_EPI = {"none": EPI_NONE, "silu_mul": EPI_SILU_MUL, "silu_mul_qfp8": EPI_SILU_MUL_QFP8,
        "topk_combine": EPI_TOPK_COMBINE, "i32_acc": EPI_I32_ACC}


class HQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


def _status_name(s: int) -> str:
    names = ["HQ_OK", "HQ_ERR_INVALID_ARG", "HQ_ERR_UNSUPPORTED", "HQ_ERR_WORKSPACE", "HQ_ERR_HIP",
             "HQ_ERR_INTERNAL"]
    return names[s] if 0 <= s < len(names) else f"HQ_ERR_{s}"


# ------------------------------------------------------------- structures --
class QuantDesc(ctypes.Structure):
    _fields_ = [("w_elem", ctypes.c_int), ("w_bits", ctypes.c_int), ("group_size", ctypes.c_int),
                ("scale", ctypes.c_int), ("zp", ctypes.c_int), ("zp_value", ctypes.c_int),
                ("act", ctypes.c_int), ("act_scale", ctypes.c_int), ("out", ctypes.c_int)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("num_experts", ctypes.c_int),
                ("q", QuantDesc)]


class Compute(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("epi", ctypes.c_int), ("mfma_in", ctypes.c_int)]


class Tuning(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int),
                ("waves", ctypes.c_int), ("split_k", ctypes.c_int), ("stages", ctypes.c_int),
                ("mfma", ctypes.c_int), ("tile_group", ctypes.c_int)]


class JitStats(ctypes.Structure):
    _fields_ = [("compiles", ctypes.c_int64), ("disk_hits", ctypes.c_int64), ("memory_hits", ctypes.c_int64),
                ("launches", ctypes.c_int64), ("compile_seconds", ctypes.c_double), ("load_seconds", ctypes.c_double)]


class AutotuneResult(ctypes.Structure):
    _fields_ = [("best", Tuning), ("best_us", ctypes.c_float), ("current_us", ctypes.c_float),
                ("candidates", ctypes.c_int)]


_TUNING_FIELDS = ("kernel", "tile_m", "tile_n", "waves", "split_k", "stages", "tile_group")


def _tuning_dict(t: Tuning) -> dict:
    return {f: int(getattr(t, f)) for f in _TUNING_FIELDS}


def w4a16(act: str = "f16", scale: Optional[str] = None, zp="fixed", zp_value: int = 8,
          out: Optional[str] = None) -> QuantDesc:
    """INT4 (group 128) weights x fp16/bf16 activations.  zp: 'fixed' or 'u4'."""
    return QuantDesc(U4, 4, 128, _DT[scale or act], ZP_FIXED if zp == "fixed" else ZP_PER_GROUP_U4,
                     zp_value, _DT[act], ASCALE_NONE, _DT[out or act])


def w8a16(act: str = "f16", scale: Optional[str] = None, zp_value: int = 128, out: Optional[str] = None) -> QuantDesc:
    """INT8 (group 128, fixed zero point) weights x fp16/bf16 activations; codes
    are uint8 [N, K], one byte per weight."""
    return QuantDesc(U8, 8, 128, _DT[scale or act], ZP_FIXED, zp_value, _DT[act], ASCALE_NONE, _DT[out or act])


def w2a16(act: str = "f16", scale: Optional[str] = None, zp_value: int = 2, out: Optional[str] = None) -> QuantDesc:
    """INT2 (group 128, fixed zero point) weights x fp16/bf16 activations; codes
    are int32 [N, K/16], sixteen 2-bit codes per word, lowest bits first."""
    return QuantDesc(U2, 2, 128, _DT[scale or act], ZP_FIXED, zp_value, _DT[act], ASCALE_NONE, _DT[out or act])


def w3a16(act: str = "f16", scale: Optional[str] = None, zp_value: int = 4, out: Optional[str] = None) -> QuantDesc:
    """INT3 (group 128, fixed zero point) weights x fp16/bf16 activations; codes
    are int32 [N, 3K/32], the dense 3-bit packing of GPTQ INT3 along K (each
    row one little-endian bit stream, code k in bits [3k, 3k+3))."""
    return QuantDesc(U3, 3, 128, _DT[scale or act], ZP_FIXED, zp_value, _DT[act], ASCALE_NONE, _DT[out or act])


def w4a16_mxint4(act: str = "bf16", out: Optional[str] = None) -> QuantDesc:
    """MXINT4 weights (two's-complement 4-bit codes times 2^-2, one E8M0 scale
    per 32 k; codes packed as INT4, scales uint8 [N, K/32]) x fp16/bf16
    activations."""
    return QuantDesc(I4, 4, 32, E8M0, ZP_NONE, 0, _DT[act], ASCALE_NONE, _DT[out or act])


def w4a16_nvfp4(act: str = "bf16", out: Optional[str] = None) -> QuantDesc:
    """NVFP4 weights (E2M1 codes packed as INT4, one E4M3 scale per 16 k as
    uint8 [N, K/16], one fp32 tensor scale) x fp16/bf16 activations.  Repack
    with scales = the tensor scale (float32 [1], or [E] for stacked weights)
    and e8m0 = the E4M3 block scales."""
    return QuantDesc(FP4_E2M1, 4, 16, FP8_E4M3, ZP_NONE, 0, _DT[act], ASCALE_NONE, _DT[out or act])


def w4a8_int(scale: str = "f16", out: str = "bf16") -> QuantDesc:
    """INT4 (group 128, zero 8) weights x int8 per-token activations."""
    return QuantDesc(U4, 4, 128, _DT[scale], ZP_FIXED, 8, INT8, ASCALE_PER_TOKEN_F32, _DT[out])


def w4a8_fp8(scale: str = "f16", zp="fixed", zp_value: int = 8, out: str = "bf16") -> QuantDesc:
    """INT4 (group 128) weights x fp8 e4m3 per-token activations."""
    return QuantDesc(U4, 4, 128, _DT[scale], ZP_FIXED if zp == "fixed" else ZP_PER_GROUP_U4, zp_value,
                     FP8_E4M3, ASCALE_PER_TOKEN_F32, _DT[out])


def w4a8_mxfp4(out: str = "bf16") -> QuantDesc:
    """MXFP4 (E2M1 + E8M0 per 32) weights x fp8 e4m3 per-token activations."""
    return QuantDesc(FP4_E2M1, 4, 32, E8M0, ZP_NONE, 0, FP8_E4M3, ASCALE_PER_TOKEN_F32, _DT[out])


def w4a4_mxfp4(out: str = "bf16") -> QuantDesc:
    """MXFP4 weights x MXFP4 activations (E2M1 codes packed two per byte along
    K; E8M0 block scales passed as a_scale in the group-major layout
    [K/128, m, 4], see mx_scales_group_major)."""
    return QuantDesc(FP4_E2M1, 4, 32, E8M0, ZP_NONE, 0, FP4_E2M1, ASCALE_MX_E8M0, _DT[out])


# ---------------------------------------------------------------- library --
_lib = None

_SIGS = {
    "hq_abi_version": (ctypes.c_int, []),
    "hq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "hq_last_error": (ctypes.c_char_p, []),
    "hq_plan_create": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(Compute), ctypes.c_int64,
                                      ctypes.POINTER(Tuning), ctypes.POINTER(ctypes.c_void_p)]),
    "hq_plan_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "hq_plan_describe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_char_p, ctypes.c_size_t]),
    "hq_plan_workspace_bytes": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.POINTER(ctypes.c_size_t)]),
    "hq_repacked_bytes": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                                         ctypes.POINTER(ctypes.c_size_t)]),
    "hq_repack": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 5 + [ctypes.c_void_p]),
    "hq_repack_host": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 5),
    "hq_time_next_launch": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "hq_moe_block_m": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]),
    "hq_moe_max_padded": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int64)]),
    "hq_moe_align": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int] +
                     [ctypes.c_void_p] * 5),
    "hq_moe_workspace_bytes": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_size_t)]),
    "hq_moe_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int] + [ctypes.c_void_p] * 11 +
                    [ctypes.c_size_t, ctypes.c_void_p]),
    "hq_moe_gemm_by_slot": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int] + [ctypes.c_void_p] * 9 +
                            [ctypes.c_size_t, ctypes.c_void_p]),
    "hq_stream_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]),
    "hq_mfma_peak": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]),
    "hq_quantize_per_token": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int] +
                              [ctypes.c_void_p] * 4),
    "hq_quantize_mxfp4": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int] + [ctypes.c_void_p] * 4),
    "hq_plan_autotune": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 6 +
                         [ctypes.c_size_t, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p,
                          ctypes.POINTER(AutotuneResult)]),
    "hq_plan_set_tuning": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(Tuning)]),
    "hq_plan_get_tuning": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(Tuning),
                                          ctypes.POINTER(ctypes.c_int)]),
    "hq_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_size_t, ctypes.c_void_p]),
    "hq_gemm_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 5 +
                        [ctypes.c_void_p]),
    "hq_plan_set_jit": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p]),
    "hq_jit_cache_key": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_char_p, ctypes.c_char_p,
                                        ctypes.c_size_t]),
    "hq_jit_get_stats": (ctypes.c_int, [ctypes.POINTER(JitStats)]),
    "hq_jit_prepare": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_char_p]),
}


def jit_stats() -> dict:
    """Counters of the run-time specialisation since the library was loaded
    (hq_jit_get_stats)."""
    st = JitStats()
    _check(lib().hq_jit_get_stats(ctypes.byref(st)))
    return {f: getattr(st, f) for f, _ in JitStats._fields_}


def lib():
    """Load libhq.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions(path: str = HEADER_PATH):
    """Names of the functions declared in include/hq.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(hq_[a-z0-9_]+)\s*\(",
                                 text, flags=re.M)))


def _check(status: int):
    if status != HQ_OK:
        raise HQError(status, lib().hq_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_TORCH_OUT = {F16: torch.float16, BF16: torch.bfloat16}
_DT_NAME = {F16: "f16", BF16: "bf16", FP8_E4M3: "fp8", INT8: "int8", FP4_E2M1: "mxfp4"}


# ------------------------------------------------------------------ plan --
def _as16(q: QuantDesc) -> QuantDesc:
    """The same weights with 16-bit activations (the output dtype's type)."""
    act = q.out if q.out in (F16, BF16) else BF16
    return QuantDesc(q.w_elem, q.w_bits, q.group_size, q.scale, q.zp, q.zp_value, act, ASCALE_NONE, q.out)


class Plan:
    """A layer description + execution choice (owns an hq_plan).

    mfma_in names the matrix-instruction operand type ('f16', 'bf16', 'fp8',
    'int8', 'fp8xfp4', 'fp4'; None: the description's).  When the library
    cannot run the description (HQ_ERR_UNSUPPORTED) and its activations are 8-
    or 4-bit, the plan is built again for the same weights with 16-bit
    activations -- the pages' fallback to a higher-precision compute type
    (Humming page on news.ditty.ir, summary) -- unless fallback=False.  Then
    `fallback` holds the reason, `quant` the description that runs and
    `requested_quant` the one asked for; `linear` takes 16-bit activations
    either way."""

    def __init__(self, n: int, k: int, quant: QuantDesc, max_m: int, epi: str = "none",
                 kind: str = "dense", num_experts: int = 1, tuning: Optional[dict] = None,
                 mfma_in: Optional[str] = None, fallback: bool = True):
        L = lib()
        self.n, self.k, self.max_m, self.num_experts = int(n), int(k), int(max_m), int(num_experts)
        self.requested_quant = quant
        self.quant = quant
        self.fallback = None
        self.epi = _EPI[epi]
        if mfma_in not in _MFMA:
            raise ValueError(f"mfma_in must be one of {sorted(k for k in _MFMA if k)}")
        tun = None
        if tuning:
            tun = Tuning(**{key: int(v) for key, v in tuning.items()})

        def create(q, mi):
            layer = LayerDesc(self.n, self.k, self.num_experts, q)
            comp = Compute(GEMM_DENSE if kind == "dense" else GEMM_GROUPED, self.epi, mi)
            h = ctypes.c_void_p()
            _check(L.hq_plan_create(ctypes.byref(layer), ctypes.byref(comp), self.max_m,
                                    ctypes.byref(tun) if tun is not None else None, ctypes.byref(h)))
            return h

        try:
            handle = create(quant, _MFMA[mfma_in])
        except HQError as e:
            if not fallback or e.status != HQ_ERR_UNSUPPORTED or quant.act in (F16, BF16) or \
                    self.epi == EPI_I32_ACC:
                raise
            q16 = _as16(quant)
            try:
                handle = create(q16, MFMA_AUTO)
            except HQError:
                raise e from None
            self.quant = q16
            self.fallback = (f"{_DT_NAME.get(quant.act, quant.act)} activations requested: {e}; running "
                             f"{_DT_NAME[q16.act]} activations")
        self._h = handle
        self._ws = {}
        self._act_buf = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.hq_plan_destroy(h)
            self._h = None

    # -- sizes ----------------------------------------------------------
    def repacked_bytes(self):
        w, m = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().hq_repacked_bytes(self._h, ctypes.byref(w), ctypes.byref(m)))
        return w.value, m.value

    def workspace_bytes(self, m: int) -> int:
        b = ctypes.c_size_t()
        _check(lib().hq_plan_workspace_bytes(self._h, int(m), ctypes.byref(b)))
        return b.value

    def describe(self, m: int) -> str:
        buf = ctypes.create_string_buffer(512)
        _check(lib().hq_plan_describe(self._h, int(m), buf, 512))
        d = buf.value.decode()
        return d if self.fallback is None else f"{d} fallback=16-bit-activations ({self.fallback})"

    def workspace(self, m: int, device) -> Optional[torch.Tensor]:
        """A zero-initialised workspace kept per device (reused across calls;
        the kernels leave it ready for the next call on the same stream)."""
        need = self.workspace_bytes(m)
        if need == 0:
            return None
        dev = torch.device(device)
        ws = self._ws.get(dev)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
            self._ws[dev] = ws
        return ws

    # -- repack ---------------------------------------------------------
    def _repack_outputs(self, device):
        wb, mb = self.repacked_bytes()
        w = torch.empty(wb, dtype=torch.uint8, device=device)
        meta = torch.empty(max(mb, 16), dtype=torch.uint8, device=device)
        return w, meta

    def repack(self, codes: torch.Tensor, scales: Optional[torch.Tensor] = None,
               zeros: Optional[torch.Tensor] = None, e8m0: Optional[torch.Tensor] = None):
        """Canonical device tensors -> (w, meta) device-layout tensors (GPU kernel)."""
        _dev(codes, "codes")
        for t, nm in ((scales, "scales"), (zeros, "zeros"), (e8m0, "e8m0")):
            if t is not None:
                _dev(t, nm)
        w, meta = self._repack_outputs(codes.device)
        zx = e8m0 if e8m0 is not None else zeros
        _check(lib().hq_repack(self._h, _ptr(codes), _ptr(scales), _ptr(zx), _ptr(w), _ptr(meta),
                               _stream_ptr(codes.device)))
        return w, meta

    def repack_host(self, codes: torch.Tensor, scales: Optional[torch.Tensor] = None,
                    zeros: Optional[torch.Tensor] = None, e8m0: Optional[torch.Tensor] = None):
        """The same permutation on CPU tensors (offline preparation)."""
        ts = [t.contiguous() if t is not None else None for t in (codes, scales, zeros, e8m0)]
        for t in ts:
            if t is not None and t.is_cuda:
                raise ValueError("repack_host takes CPU tensors")
        codes, scales, zeros, e8m0 = ts
        w, meta = self._repack_outputs("cpu")
        zx = e8m0 if e8m0 is not None else zeros
        _check(lib().hq_repack_host(self._h, _ptr(codes), _ptr(scales), _ptr(zx), _ptr(w), _ptr(meta)))
        return w, meta

    # -- GEMM -----------------------------------------------------------
    def gemm(self, a: torch.Tensor, w: torch.Tensor, meta: torch.Tensor, a_scale: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
        """out[m, n] = A . W_deq^T (see include/hq.h, hq_gemm)."""
        _dev(a, "a"), _dev(w, "w"), _dev(meta, "meta")
        act4 = self.quant.act == FP4_E2M1
        if a_scale is not None:
            _dev(a_scale, "a_scale")
            if a_scale.dtype != (torch.uint8 if act4 else torch.float32):
                raise ValueError("a_scale must be uint8 E8M0 [m, k/32] (MXFP4 activations) or float32 [m]")
        m = a.shape[0]
        if act4:  # MXFP4 codes two per byte: [m, k/2] bytes (or [m, k/8] int32 words)
            if a.dim() != 2 or a.shape[1] * a.element_size() != self.k // 2:
                raise ValueError(f"a must hold [m, {self.k // 2}] bytes of packed MXFP4 codes")
        elif a.dim() != 2 or a.shape[1] != self.k:
            raise ValueError(f"a must be [m, {self.k}]")
        if out is None:
            if self.epi == EPI_I32_ACC:
                out = torch.empty((m, self.n, self.k // 128), dtype=torch.int32, device=a.device)
            else:
                out = torch.empty((m, self.n), dtype=_TORCH_OUT[self.quant.out], device=a.device)
        _dev(out, "out")
        if ws is None:
            ws = self.workspace(m, a.device)
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(lib().hq_gemm(self._h, m, _ptr(a), _ptr(a_scale), _ptr(w), _ptr(meta), _ptr(out), _ptr(ws),
                             ws_bytes, _stream_ptr(a.device)))
        return out


    def linear(self, x: torch.Tensor, w: torch.Tensor, meta: torch.Tensor, out: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None) -> torch.Tensor:
        """out = x . W_deq^T for 16-bit activations x [m, k]: a plan that runs
        8-bit activations quantises x per token first (hq_quantize_per_token:
        fp8 e4m3 or int8), one that runs MXFP4 activations block-quantises it
        (hq_quantize_mxfp4), a 16-bit plan -- including one that fell back --
        multiplies x as it is.  Every step is a library kernel on x's stream;
        the activation codes live in a buffer kept per device and m."""
        _dev(x, "x")
        if x.dtype not in (torch.float16, torch.bfloat16) or x.dim() != 2 or x.shape[1] != self.k:
            raise ValueError(f"x must be fp16 / bf16 [m, {self.k}]")
        q = self.quant
        if q.act in (F16, BF16):
            if x.dtype != _TORCH_OUT[q.act]:
                raise ValueError(f"this plan multiplies {_DT_NAME[q.act]} activations")
            return self.gemm(x, w, meta, out=out, ws=ws)
        m = x.shape[0]
        key = (x.device, m)
        buf = self._act_buf.get(key)
        if q.act == FP4_E2M1:
            if buf is None:
                buf = (torch.empty((m, self.k // 2), dtype=torch.uint8, device=x.device),
                       torch.empty((self.k // 128, m, 4), dtype=torch.uint8, device=x.device))
                self._act_buf[key] = buf
            codes, sc = quantize_mxfp4(x, codes=buf[0], e8m0=buf[1])
        else:
            kind = "fp8" if q.act == FP8_E4M3 else "int8"
            if buf is None:
                buf = (torch.empty((m, self.k), dtype=torch.uint8 if kind == "fp8" else torch.int8, device=x.device),
                       torch.empty(m, dtype=torch.float32, device=x.device))
                self._act_buf[key] = buf
            codes, sc = quantize_per_token(x, kind, codes=buf[0], scales=buf[1])
        return self.gemm(codes, w, meta, a_scale=sc, out=out, ws=ws)

    # -- measured execution choices --------------------------------------
    def autotune(self, a: torch.Tensor, w: torch.Tensor, meta: torch.Tensor, a_scale: Optional[torch.Tensor] = None,
                 reps: int = 10, flush_bytes: int = 512 << 20, max_ws_bytes: int = 512 << 20) -> dict:
        """Time the candidate execution choices for m = a.shape[0] rows on these
        buffers and install the fastest for that m (see hq_plan_autotune).
        Returns {"tuning", "best_us", "current_us", "candidates"}."""
        _dev(a, "a"), _dev(w, "w"), _dev(meta, "meta")
        if a_scale is not None:
            _dev(a_scale, "a_scale")
        m = a.shape[0]
        out = torch.empty((m, self.n), dtype=_TORCH_OUT.get(self.quant.out, torch.float16), device=a.device)
        if self.epi == EPI_I32_ACC:
            out = torch.empty((m, self.n, self.k // 128), dtype=torch.int32, device=a.device)
        ws_bytes = min(int(max_ws_bytes), 8 * m * self.n * 4)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=a.device)
        res = AutotuneResult()
        _check(lib().hq_plan_autotune(self._h, m, _ptr(a), _ptr(a_scale), _ptr(w), _ptr(meta), _ptr(out), _ptr(ws),
                                      ws_bytes, int(reps), int(flush_bytes), _stream_ptr(a.device),
                                      ctypes.byref(res)))
        return {"tuning": _tuning_dict(res.best), "best_us": float(res.best_us),
                "current_us": float(res.current_us), "candidates": int(res.candidates)}

    def set_jit(self, enable: bool = True, cache_dir: Optional[str] = None):
        """Run-time specialised kernels for this dense plan (hq_plan_set_jit):
        each call's shape compiled once by hipRTC, code objects cached on disk
        under cache_dir (None: the library's default directory)."""
        _check(lib().hq_plan_set_jit(self._h, 1 if enable else 0,
                                     None if cache_dir is None else os.fsencode(cache_dir)))

    def jit_cache_key(self, m: int, arch: str = "gfx950") -> str:
        """The code-object cache key of the kernel a call with m rows runs under
        run-time specialisation (hq_jit_cache_key; host only)."""
        buf = ctypes.create_string_buffer(128)
        _check(lib().hq_jit_cache_key(self._h, int(m), arch.encode(), buf, len(buf)))
        return buf.value.decode()

    def jit_prepare(self, m: int, arch: str = "gfx950"):
        """Compile the m-row kernel of run-time specialisation into the plan's
        code-object cache without a device (hq_jit_prepare)."""
        _check(lib().hq_jit_prepare(self._h, int(m), arch.encode()))

    def set_tuning(self, m: int, tuning: Optional[dict]):
        """Install a tuning for exactly m rows (None removes m's entry)."""
        t = None if tuning is None else Tuning(**{f: int(tuning.get(f, 0)) for f in _TUNING_FIELDS})
        _check(lib().hq_plan_set_tuning(self._h, int(m), None if t is None else ctypes.byref(t)))

    def get_tuning(self, m: int):
        """(resolved tuning dict for m rows, whether it comes from the table)."""
        t, flag = Tuning(), ctypes.c_int(0)
        _check(lib().hq_plan_get_tuning(self._h, int(m), ctypes.byref(t), ctypes.byref(flag)))
        return _tuning_dict(t), bool(flag.value)

    def tuning_key(self, m: int, device) -> str:
        """Cache key of m rows of this plan on `device`: format, shape, GPU, rows."""
        q = self.quant
        fmt = "-".join(str(int(getattr(q, f))) for f, _ in QuantDesc._fields_)
        name = torch.cuda.get_device_name(torch.device(device)).replace("|", "/")
        return f"{fmt}|epi{self.epi}|n{self.n}|k{self.k}|{name}|abi{lib().hq_abi_version()}|m{int(m)}"


class TuningCache:
    """Measured execution choices kept across processes: a JSON file that maps
    Plan.tuning_key(m, device) to a resolved tuning."""

    def __init__(self, path: str):
        self.path = path
        self.entries = {}
        if os.path.exists(path):
            with open(path) as f:
                self.entries = json.load(f)

    def save(self):
        tmp = self.path + ".tmp"
        with open(tmp, "w") as f:
            json.dump(self.entries, f, indent=1, sort_keys=True)
        os.replace(tmp, self.path)

    def apply(self, plan: Plan, device) -> int:
        """Install every cached tuning of this plan on `device`; returns how many."""
        prefix = plan.tuning_key(0, device)[:-1]  # everything but the row count
        n = 0
        for key, t in self.entries.items():
            if key.startswith(prefix) and key[len(prefix):].isdigit() and 1 <= int(key[len(prefix):]) <= plan.max_m:
                plan.set_tuning(int(key[len(prefix):]), t)
                n += 1
        return n

    def tune(self, plan: Plan, a: torch.Tensor, w: torch.Tensor, meta: torch.Tensor,
             a_scale: Optional[torch.Tensor] = None, **kw) -> dict:
        """The cached tuning for a's rows if there is one (installed), else an
        autotune run whose result is installed and saved."""
        key = plan.tuning_key(a.shape[0], a.device)
        if key in self.entries:
            plan.set_tuning(a.shape[0], self.entries[key])
            return {"tuning": dict(self.entries[key]), "cached": True}
        r = plan.autotune(a, w, meta, a_scale, **kw)
        self.entries[key] = r["tuning"]
        self.save()
        return dict(r, cached=False)


def stream_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int, nbytes: Optional[int] = None):
    """Bandwidth probe: read `nbytes` (default all) of `buf` once (see hq_stream_read)."""
    _dev(buf, "buf"), _dev(sink, "sink")
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    _check(lib().hq_stream_read(_ptr(buf), n, _ptr(sink), int(workgroups), _stream_ptr(buf.device)))


def mfma_peak(kind: int, sink: torch.Tensor, workgroups: int = 1024, iters: int = 2000) -> float:
    """Matrix-core throughput probe (see hq_mfma_peak): one launch of `kind`
    (PEAK_F16 .. PEAK_INT8) on the stream of `sink`; returns its operations."""
    _dev(sink, "sink")
    fl = ctypes.c_double()
    _check(lib().hq_mfma_peak(int(kind), int(workgroups), int(iters), _ptr(sink), ctypes.byref(fl),
                              _stream_ptr(sink.device)))
    return fl.value


def quantize_per_token(x: torch.Tensor, out: str = "fp8", codes: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None):
    """Per-row 8-bit quantisation of fp16 / bf16 activations [m, k] (see
    hq_quantize_per_token): scales = max|row| / Q, codes = RNE(x / scale).
    out "fp8" gives uint8 e4m3 codes (Q = 448), "int8" int8 codes (Q = 127).
    Returns (codes [m, k], scales fp32 [m]), the (a, a_scale) of a W4A8 GEMM."""
    _dev(x, "x")
    if x.dim() != 2 or x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x must be fp16 / bf16 [m, k]")
    if out not in ("fp8", "int8"):
        raise ValueError("out must be 'fp8' or 'int8'")
    m, k = x.shape
    cdt = torch.uint8 if out == "fp8" else torch.int8
    if codes is None:
        codes = torch.empty((m, k), dtype=cdt, device=x.device)
    if scales is None:
        scales = torch.empty(m, dtype=torch.float32, device=x.device)
    _dev(codes, "codes"), _dev(scales, "scales")
    if codes.shape != (m, k) or codes.element_size() != 1 or scales.numel() != m or scales.dtype != torch.float32:
        raise ValueError("codes must be 1-byte [m, k] and scales fp32 [m]")
    _check(lib().hq_quantize_per_token(m, k, BF16 if x.dtype == torch.bfloat16 else F16,
                                       FP8_E4M3 if out == "fp8" else INT8, _ptr(x), _ptr(codes), _ptr(scales),
                                       _stream_ptr(x.device)))
    return codes, scales


def mx_scales_group_major(e8m0_rows: torch.Tensor) -> torch.Tensor:
    """Row-major E8M0 block scales [m, K/32] -> the group-major words
    [K/128, m, 4] that a W4A4 GEMM reads (a copy; runs where the tensor is)."""
    m, kb = e8m0_rows.shape
    return e8m0_rows.reshape(m, kb // 4, 4).transpose(0, 1).contiguous()


def quantize_mxfp4(x: torch.Tensor, codes: Optional[torch.Tensor] = None, e8m0: Optional[torch.Tensor] = None):
    """MXFP4 block quantisation of fp16 / bf16 activations [m, k] (see
    hq_quantize_mxfp4).  Returns (codes uint8 [m, k/2], e8m0 uint8
    [k/128, m, 4] group-major), the (a, a_scale) of a W4A4 GEMM."""
    _dev(x, "x")
    if x.dim() != 2 or x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x must be fp16 / bf16 [m, k]")
    m, k = x.shape
    if codes is None:
        codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if e8m0 is None:
        e8m0 = torch.empty((k // 128, m, 4), dtype=torch.uint8, device=x.device)
    _dev(codes, "codes"), _dev(e8m0, "e8m0")
    if codes.numel() * codes.element_size() != m * (k // 2) or e8m0.numel() != m * (k // 32) or \
            e8m0.dtype != torch.uint8:
        raise ValueError("codes must hold [m, k/2] bytes and e8m0 be uint8 [k/128, m, 4]")
    _check(lib().hq_quantize_mxfp4(m, k, BF16 if x.dtype == torch.bfloat16 else F16, _ptr(x), _ptr(codes),
                                   _ptr(e8m0), _stream_ptr(x.device)))
    return codes, e8m0


# ------------------------------------------------------------------- MoE --
def moe_max_padded(t: int, topk: int, num_experts: int, block_m: int) -> int:
    v = ctypes.c_int64()
    _check(lib().hq_moe_max_padded(int(t), int(topk), int(num_experts), int(block_m), ctypes.byref(v)))
    return v.value


def moe_align(topk_ids: torch.Tensor, num_experts: int, block_m: int):
    """Token sort / align by expert (see hq_moe_align).  topk_ids: int32 [t, topk] on the GPU.
    Returns (sorted_ids, block_expert, num_padded) device int32 tensors."""
    _dev(topk_ids, "topk_ids")
    if topk_ids.dtype != torch.int32 or topk_ids.dim() != 2:
        raise ValueError("topk_ids must be int32 [t, topk]")
    t, topk = topk_ids.shape
    mp = moe_max_padded(t, topk, num_experts, block_m)
    dev = topk_ids.device
    sorted_ids = torch.empty(mp, dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(mp // block_m, 1), dtype=torch.int32, device=dev)
    num_padded = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib().hq_moe_align(t, topk, int(num_experts), int(block_m), _ptr(topk_ids), _ptr(sorted_ids),
                              _ptr(block_expert), _ptr(num_padded), _stream_ptr(dev)))
    return sorted_ids, block_expert, num_padded


class MoePlan(Plan):
    """A grouped plan: num_experts weights of [n, k]; epi one of 'silu_mul',
    'silu_mul_qfp8' (gate_up), 'topk_combine' (down) or 'none'."""

    def __init__(self, n: int, k: int, quant: QuantDesc, num_experts: int, max_t: int, epi: str,
                 tuning: Optional[dict] = None, mfma_in: Optional[str] = None, fallback: bool = False):
        super().__init__(n, k, quant, max_m=max_t, epi=epi, kind="grouped", num_experts=num_experts, tuning=tuning,
                         mfma_in=mfma_in, fallback=fallback)

    def describe(self, t: int, topk: int = 1) -> str:
        """The kernel a grouped call with t tokens of topk slots launches."""
        return super().describe(int(t) * int(topk))

    def block_m(self, t: int, topk: int) -> int:
        v = ctypes.c_int()
        _check(lib().hq_moe_block_m(self._h, int(t), int(topk), ctypes.byref(v)))
        return v.value

    def moe_workspace(self, t: int, topk: int, device) -> Optional[torch.Tensor]:
        b = ctypes.c_size_t()
        _check(lib().hq_moe_workspace_bytes(self._h, int(t), int(topk), ctypes.byref(b)))
        if b.value == 0:
            return None
        dev = torch.device(device)
        ws = self._ws.get(dev)
        if ws is None or ws.numel() < b.value:
            ws = torch.zeros(b.value, dtype=torch.uint8, device=dev)
            self._ws[dev] = ws
        return ws

    def moe_gemm(self, a: torch.Tensor, t: int, topk: int, sorted_ids: torch.Tensor, block_expert: torch.Tensor,
                 num_padded: torch.Tensor, w: torch.Tensor, meta: torch.Tensor, a_scale=None, topk_w=None,
                 out=None, out_scale=None, ws=None):
        for x, nm in ((a, "a"), (sorted_ids, "sorted_ids"), (block_expert, "block_expert"),
                      (num_padded, "num_padded"), (w, "w"), (meta, "meta")):
            _dev(x, nm)
        dev = a.device
        bm = self.block_m(t, topk)
        need = moe_max_padded(t, topk, self.num_experts, bm)
        if sorted_ids.numel() < need or block_expert.numel() < max(need // bm, 1):
            raise ValueError(f"sorted_ids / block_expert are smaller than an alignment with block_m={bm} "
                             f"for t={t}, topk={topk} needs ({need}, {need // bm}); align with block_m(t, topk)")
        mp = sorted_ids.numel()
        if out is None:
            if self.epi == EPI_TOPK_COMBINE:
                out = torch.empty((t, self.n), dtype=_TORCH_OUT[self.quant.out], device=dev)
            elif self.epi == EPI_SILU_MUL_QFP8:
                out = torch.empty((mp, self.n // 2), dtype=torch.uint8, device=dev)
            elif self.epi == EPI_SILU_MUL:
                out = torch.empty((mp, self.n // 2), dtype=_TORCH_OUT[self.quant.out], device=dev)
            else:
                out = torch.empty((mp, self.n), dtype=_TORCH_OUT[self.quant.out], device=dev)
        if self.epi == EPI_SILU_MUL_QFP8 and out_scale is None:
            out_scale = torch.empty(mp, dtype=torch.float32, device=dev)
        if ws is None:
            ws = self.moe_workspace(t, topk, dev)
        ws_bytes = 0 if ws is None else ws.numel()
        _check(lib().hq_moe_gemm(self._h, int(t), int(topk), _ptr(a), _ptr(a_scale), _ptr(sorted_ids),
                                 _ptr(block_expert), _ptr(num_padded), _ptr(topk_w), _ptr(w), _ptr(meta), _ptr(out),
                                 _ptr(out_scale), _ptr(ws), ws_bytes, _stream_ptr(dev)))
        return (out, out_scale) if self.epi == EPI_SILU_MUL_QFP8 else out

    def moe_gemm_by_slot(self, a: torch.Tensor, t: int, topk: int, topk_ids: torch.Tensor, w: torch.Tensor,
                         meta: torch.Tensor, a_scale=None, topk_w=None, out=None, out_scale=None, ws=None):
        """hq_moe_gemm_by_slot: the grouped GEMM with rows indexed by routed
        slot (no alignment).  gate_up returns [t*topk, n/2] (fp8: codes and
        per-slot scales); down takes those slot rows and returns y [t, n]."""
        for x, nm in ((a, "a"), (topk_ids, "topk_ids"), (w, "w"), (meta, "meta")):
            _dev(x, nm)
        dev = a.device
        slots = int(t) * int(topk)
        if topk_ids.numel() < slots:
            raise ValueError(f"topk_ids holds {topk_ids.numel()} ids, t * topk = {slots}")
        if out is None:
            if self.epi == EPI_TOPK_COMBINE:
                out = torch.empty((t, self.n), dtype=_TORCH_OUT[self.quant.out], device=dev)
            elif self.epi == EPI_SILU_MUL_QFP8:
                out = torch.empty((slots, self.n // 2), dtype=torch.uint8, device=dev)
            elif self.epi == EPI_SILU_MUL:
                out = torch.empty((slots, self.n // 2), dtype=_TORCH_OUT[self.quant.out], device=dev)
            else:
                out = torch.empty((slots, self.n), dtype=_TORCH_OUT[self.quant.out], device=dev)
        if self.epi == EPI_SILU_MUL_QFP8 and out_scale is None:
            out_scale = torch.empty(slots, dtype=torch.float32, device=dev)
        if ws is None and self.epi == EPI_SILU_MUL_QFP8:
            ws = self.moe_workspace(t, topk, dev)
        ws_bytes = 0 if ws is None else ws.numel()
        _check(lib().hq_moe_gemm_by_slot(self._h, int(t), int(topk), _ptr(a), _ptr(a_scale), _ptr(topk_ids),
                                         _ptr(topk_w), _ptr(w), _ptr(meta), _ptr(out), _ptr(out_scale), _ptr(ws),
                                         ws_bytes, _stream_ptr(dev)))
        return (out, out_scale) if self.epi == EPI_SILU_MUL_QFP8 else out


# Routed slots (t * topk) up to which moe_layer takes the unaligned by-slot
# path: measured on MI355X (256 experts, top 8, H = 7168, I = 256) it is the
# faster one up to 32 slots and level with the aligned path at 64, where an
# expert picked by several slots starts to be read once per slot.
# routed slots up to which moe_layer takes the by-slot path: the measured
# crossover on MI355X (256 experts, top 8, H = 7168, I = 256, graph-timed
# layers): bf16 by slot against aligned 60.7 / 71.0 us at T = 12 and 82.9 /
# 85.4 us at T = 16; fp8 64.0 / 66.3 us at T = 12 and 78.0 / 76.3 us at T = 16
MOE_BY_SLOT_MAX_SLOTS = 128
MOE_BY_SLOT_MAX_SLOTS_FP8 = 96


def moe_uses_by_slot(t: int, topk: int, fp8: bool = False) -> bool:
    """Whether moe_layer runs a call of t tokens routed to topk experts each
    (fp8: W4A8-FP8 activations) through hq_moe_gemm_by_slot (else the aligned
    hq_moe_align + hq_moe_gemm)."""
    limit = MOE_BY_SLOT_MAX_SLOTS_FP8 if fp8 else MOE_BY_SLOT_MAX_SLOTS
    return 0 < int(t) * int(topk) <= limit


def moe_layer(gate_up: "MoePlan", down: "MoePlan", x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
              w1: torch.Tensor, m1: torch.Tensor, w2: torch.Tensor, m2: torch.Tensor, x_scale=None,
              by_slot: Optional[bool] = None) -> torch.Tensor:
    """One MoE layer, y [t, n_down]: gate_up (SiLU * up, or with the fp8
    requant) then down with the top-k combine, on the by-slot path for
    decode-sized calls (moe_uses_by_slot) and the aligned path otherwise;
    `by_slot` forces one.  x: [t, k] activations (fp8 codes with x_scale for
    W4A8); topk_ids int32 / topk_w fp32 [t, topk] on the GPU."""
    t, topk = topk_ids.shape
    if down.epi != EPI_TOPK_COMBINE or gate_up.epi not in (EPI_SILU_MUL, EPI_SILU_MUL_QFP8):
        raise ValueError("moe_layer takes a gate_up plan (silu_mul / silu_mul_qfp8) and a topk_combine plan")
    fp8 = gate_up.epi == EPI_SILU_MUL_QFP8
    if by_slot is None:
        by_slot = moe_uses_by_slot(t, topk, fp8)
    if by_slot:
        r = gate_up.moe_gemm_by_slot(x, t, topk, topk_ids, w1, m1, a_scale=x_scale)
        act, scl = r if fp8 else (r, None)
        return down.moe_gemm_by_slot(act, t, topk, topk_ids, w2, m2, a_scale=scl, topk_w=topk_w)
    bm = gate_up.block_m(t, topk)
    if down.block_m(t, topk) != bm:
        raise ValueError("the gate_up and down plans must share one alignment block size (equal tuning)")
    sid, bex, npad = moe_align(topk_ids, gate_up.num_experts, bm)
    r = gate_up.moe_gemm(x, t, topk, sid, bex, npad, w1, m1, a_scale=x_scale)
    act, scl = r if fp8 else (r, None)
    return down.moe_gemm(act, t, topk, sid, bex, npad, w2, m2, a_scale=scl, topk_w=topk_w)
