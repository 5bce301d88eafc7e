// Second pass of a K split over workgroups: every split stored its fp32
// partial tile [M][N]; the output is the sum of the splits in index order,
// rounded once (RNE) to fp16 / bf16.  No device-wide fence or counter is
// needed, and the result does not depend on which workgroup finished first.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.h"
#include "hq_internal.h"
#include "launch.h"

namespace hq {

// Four consecutive outputs per thread (M * N is a multiple of 16).
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float4* __restrict__ part, int splits,
                                                            int64_t mn4, uint2* __restrict__ out, int out_bf16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn4; i += (int64_t)gridDim.x * blockDim.x) {
    float4 v = part[i];
    for (int s = 1; s < splits; ++s) {
      const float4 w = part[(int64_t)s * mn4 + i];
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    const uint32_t h0 = out_bf16 ? float_to_bf16_bits(v.x) : float_to_f16_bits(v.x);
    const uint32_t h1 = out_bf16 ? float_to_bf16_bits(v.y) : float_to_f16_bits(v.y);
    const uint32_t h2 = out_bf16 ? float_to_bf16_bits(v.z) : float_to_f16_bits(v.z);
    const uint32_t h3 = out_bf16 ? float_to_bf16_bits(v.w) : float_to_f16_bits(v.w);
    out[i] = uint2{h0 | (h1 << 16), h2 | (h3 << 16)};
  }
}

// ---------------------------------------------------------------------------
// Library-owned scratch for hq_gemm_noalloc: the split-K partials of a call
// that must not allocate live in this file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  In host code
// the name `scratch` is only a host-side stand-in, never a device address:
// the address is looked up once per device with hipGetSymbolAddress, with
// that device current, and only that address is handed to kernels.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return (int)hipSuccess;
}

int launch_splitk_reduce(const float* part, int splits, int64_t mn, void* out, int out_bf16, void* stream) {
  const int64_t mn4 = mn / 4;
  int64_t blocks = (mn4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  return (int)launch_timed(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0,
                           static_cast<hipStream_t>(stream), reinterpret_cast<const float4*>(part), splits, mn4,
                           static_cast<uint2*>(out), out_bf16);
}

}  // namespace hq
