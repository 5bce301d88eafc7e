"""GPU checks of the measurement probes (not part of the GEMM): the
matrix-core throughput probe's operation count against the published dense
peaks of MI355X (a rate above the peak would mean a miscounted launch), and
the streaming-read probe's rate against the HBM peak."""
import ctypes
import sys

import pytest
import torch

import bit_quantized_gemm_repack_amd as hq

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# MI355X published dense peaks (TFLOP/s, TOP/s for int8); the mixed fp8 x fp4
# form is bounded by the fp4 rate
PEAKS = {hq.PEAK_F16: 2500.0, hq.PEAK_BF16: 2500.0, hq.PEAK_FP8: 5000.0, hq.PEAK_FP8_FP4: 10100.0,
         hq.PEAK_FP4: 10100.0, hq.PEAK_INT8: 5000.0}


def _log(msg):
    print(f"[probe] {msg}", file=sys.stderr, flush=True)


def _events():
    L = hq.lib()
    hip = None
    for line in open("/proc/self/maps"):
        if "libamdhip64" in line:
            hip = ctypes.CDLL(line.split()[-1])
            break
    assert hip is not None
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return L, hip


@pytest.mark.parametrize("kind", sorted(PEAKS))
def test_mfma_probe_rate_within_published_peak(kind):
    _log(f"mfma probe kind={kind}")
    L, hip = _events()
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    hq.mfma_peak(kind, sink, 1024, 200)
    a, b = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(a)) == 0 and hip.hipEventCreate(ctypes.byref(b)) == 0
    hq._check(L.hq_time_next_launch(a, b))
    flops = hq.mfma_peak(kind, sink, 1024, 2000)
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    hip.hipEventDestroy(a)
    hip.hipEventDestroy(b)
    rate = flops / (ms.value * 1e-3) / 1e12
    _log(f"kind={kind}: {rate:.1f} TFLOP/s over {ms.value * 1e3:.1f} us")
    assert flops == 1024 * 4 * 2000 * 4 * 2 * 16 * 16 * {hq.PEAK_F16: 32, hq.PEAK_BF16: 32, hq.PEAK_INT8: 64}.get(kind, 128)
    assert 0 < rate <= 1.05 * PEAKS[kind]
    assert int(sink.item()) == 0  # the sink is never written


def test_stream_read_rate_within_hbm_peak():
    _log("stream read 1 GiB")
    L, hip = _events()
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    hq.stream_read(buf, sink, 2048)
    a, b = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(a)) == 0 and hip.hipEventCreate(ctypes.byref(b)) == 0
    hq._check(L.hq_time_next_launch(a, b))
    hq.stream_read(buf, sink, 2048)
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    hip.hipEventDestroy(a)
    hip.hipEventDestroy(b)
    gbs = (1 << 30) / (ms.value * 1e-3) / 1e9
    _log(f"stream read: {gbs:.0f} GB/s")
    assert 0 < gbs <= 8000 * 1.05
