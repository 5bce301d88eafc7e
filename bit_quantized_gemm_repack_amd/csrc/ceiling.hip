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

int launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, void* stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  return (int)launch_timed(stream_read_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                           static_cast<const u4_t*>(buf), n16, sink);
}

}  // namespace hq
