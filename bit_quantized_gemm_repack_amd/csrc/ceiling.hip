// Attainable-bandwidth probe: a plain streaming read of a device buffer with
// 16-byte loads (the access pattern of the weight stream in the GEMMs), used
// to put the GEMM's achieved bandwidth next to what a pure read reaches for
// the same number of bytes on this chip.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "hq_internal.h"
#include "launch.h"

namespace hq {

__global__ void __launch_bounds__(256) stream_read_kernel(const u4_t* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u4_t a = __builtin_nontemporal_load(buf + i);
    const u4_t b = __builtin_nontemporal_load(buf + i + stride);
    const u4_t c = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u4_t d = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^
           d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u4_t a = __builtin_nontemporal_load(buf + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; practically never stores
}

// Matrix-core throughput probe: every wave runs `iters` rounds of kChains
// independent matrix instructions of one type on register operands (no
// memory traffic), so the sustained rate of that type on this chip (its
// clock under matrix load included) can be set beside the GEMMs' rates.
constexpr int kPeakChains = 4;
constexpr int kPeakWaves = 4;

template <int DT>
__global__ void __launch_bounds__(64 * kPeakWaves) mfma_peak_kernel(int iters, uint32_t* __restrict__ sink) {
#if defined(__HIP_DEVICE_COMPILE__)  // device-only builtins; the host pass needs only the stub
  const uint32_t odd = threadIdx.x & 1u;
  float total = 0.f;
  if constexpr (DT == HQ_PEAK_INT8) {
    const int one = (int)opaque_vgpr(0x01010101u + odd);  // int8 ones (and a two)
    const i4_t a = i4_t{one, one, one, one};
    i4_t acc[kPeakChains] = {};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < kPeakChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c) total += (float)(acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3]);
  } else if constexpr (DT == HQ_PEAK_F16 || DT == HQ_PEAK_BF16) {
    constexpr bool F16 = DT == HQ_PEAK_F16;
    const uint32_t one = opaque_vgpr((F16 ? 0x3C003C00u : 0x3F803F80u) + odd);  // 1.0 (and a little more)
    const u4_t a = u4_t{one, one, one, one};
    f4_t acc[kPeakChains] = {};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < kPeakChains; ++c) acc[c] = mfma_16x16x32<F16>(a, a, acc[c]);
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c) total += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else {
    // scaled 16x16x128: fp8 (e4m3 1.0 = 0x38) and / or fp4 (e2m1 1.0 = 0x2)
    constexpr int FA = DT == HQ_PEAK_FP4 ? 4 : 0;
    constexpr int FB = DT == HQ_PEAK_FP8 ? 0 : 4;
    const int w8 = (int)opaque_vgpr(0x38383838u + odd), w4 = (int)opaque_vgpr(0x22222222u + odd);
    const int wa = FA == 4 ? w4 : w8, wb = FB == 4 ? w4 : w8;
    const i8_t a = FA == 4 ? i8_t{wa, wa, wa, wa, 0, 0, 0, 0} : i8_t{wa, wa, wa, wa, wa, wa, wa, wa};
    const i8_t b = FB == 4 ? i8_t{wb, wb, wb, wb, 0, 0, 0, 0} : i8_t{wb, wb, wb, wb, wb, wb, wb, wb};
    f4_t acc[kPeakChains] = {};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < kPeakChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], FA, FB, 0, 127, 0, 127);
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c) total += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  }
  if (__float_as_uint(total) == 0x7F800001u) sink[0] = __float_as_uint(total);  // keeps the work; never true
#endif
}

int launch_mfma_peak(int dtype, int workgroups, int iters, uint32_t* sink, void* stream) {
  const dim3 grid((unsigned)workgroups), block(64 * kPeakWaves);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case HQ_PEAK_F16: return (int)launch_timed(mfma_peak_kernel<HQ_PEAK_F16>, grid, block, 0, s, iters, sink);
    case HQ_PEAK_BF16: return (int)launch_timed(mfma_peak_kernel<HQ_PEAK_BF16>, grid, block, 0, s, iters, sink);
    case HQ_PEAK_FP8: return (int)launch_timed(mfma_peak_kernel<HQ_PEAK_FP8>, grid, block, 0, s, iters, sink);
    case HQ_PEAK_FP8_FP4:
      return (int)launch_timed(mfma_peak_kernel<HQ_PEAK_FP8_FP4>, grid, block, 0, s, iters, sink);
    case HQ_PEAK_FP4: return (int)launch_timed(mfma_peak_kernel<HQ_PEAK_FP4>, grid, block, 0, s, iters, sink);
    case HQ_PEAK_INT8: return (int)launch_timed(mfma_peak_kernel<HQ_PEAK_INT8>, grid, block, 0, s, iters, sink);
  }
  return (int)hipErrorInvalidValue;
}

// Operations of one probe launch: waves x rounds x chains x one instruction's
// 2 * 16 * 16 * K.
double mfma_peak_flops(int dtype, int workgroups, int iters) {
  const double per = dtype == HQ_PEAK_F16 || dtype == HQ_PEAK_BF16 ? 2.0 * 16 * 16 * 32
                     : dtype == HQ_PEAK_INT8                      ? 2.0 * 16 * 16 * 64
                                                                  : 2.0 * 16 * 16 * 128;
  return per * (double)workgroups * kPeakWaves * (double)iters * kPeakChains;
}

int launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, void* stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  return (int)launch_timed(stream_read_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                           static_cast<const u4_t*>(buf), n16, sink);
}

}  // namespace hq
