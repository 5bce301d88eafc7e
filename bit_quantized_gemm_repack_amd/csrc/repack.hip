// Offline weight repack on the GPU: canonical codes / scales / zero points /
// E8M0 scales -> the fragment layout described in hq_internal.h.
//
// This is the format conversion into the library's single standard
// description (Humming page on news.ditty.ir, summary: every supported
// format is converted into one standard form whose weight, scale and zero
// point are described separately).  It is a pure bit permutation: every
// output word gathers its 8 nibbles from the canonical matrix, so the
// kernel is a gather with one thread per output word.  It runs once per
// weight load and is not on the GEMM's timed path.
#include <hip/hip_runtime.h>

#include "hq_internal.h"

namespace hq {

__global__ void repack_codes_kernel(const uint32_t* __restrict__ codes, uint32_t* __restrict__ out,
                                    int64_t K, int fmt, int64_t words_per_expert, int64_t total_words,
                                    int64_t canon_words_per_expert) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_words;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / words_per_expert;
    const int64_t widx = i - e * words_per_expert;
    out[i] = repack_word(codes + e * canon_words_per_expert, K, fmt, widx);
  }
}

__global__ void repack_codes8_kernel(const uint8_t* __restrict__ codes, uint32_t* __restrict__ out, int64_t K,
                                     int64_t words_per_expert, int64_t total_words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_words;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / words_per_expert;
    const int64_t widx = i - e * words_per_expert;
    out[i] = repack_word8(codes + e * words_per_expert * 4, K, widx);
  }
}

__global__ void repack_codes2_kernel(const uint32_t* __restrict__ codes, uint32_t* __restrict__ out, int64_t K,
                                     int64_t words_per_expert, int64_t total_words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_words;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / words_per_expert;
    const int64_t widx = i - e * words_per_expert;
    out[i] = repack_word2(codes + e * words_per_expert, K, widx);
  }
}

__global__ void repack_codes3_kernel(const uint32_t* __restrict__ codes, uint32_t* __restrict__ out, int64_t K,
                                     int64_t words_per_expert, int64_t total_words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_words;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / words_per_expert;
    const int64_t widx = i - e * words_per_expert;
    out[i] = repack_word3(codes + e * words_per_expert, K, widx);
  }
}

__global__ void repack_scales_kernel(const uint16_t* __restrict__ scales, uint16_t* __restrict__ out,
                                     int64_t G, int64_t per_expert, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / per_expert;
    const int64_t eidx = i - e * per_expert;
    out[i] = scales[e * per_expert + scale_src_index(G, eidx)];
  }
}

__global__ void repack_zeros_kernel(const uint8_t* __restrict__ zeros, uint32_t* __restrict__ out,
                                    int64_t G, int64_t words_per_expert, int64_t canon_per_expert,
                                    int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / words_per_expert;
    const int64_t widx = i - e * words_per_expert;
    out[i] = zeros_word(zeros + e * canon_per_expert, G, widx);
  }
}

__global__ void repack_e8m0_kernel(const uint8_t* __restrict__ e8, uint8_t* __restrict__ out, int64_t K,
                                   int64_t per_expert, int64_t total, int cols) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / per_expert;
    const int64_t eidx = i - e * per_expert;
    out[i] = e8[e * per_expert + (cols ? e8m0_cols_src_index(K, eidx) : e8m0_src_index(K, eidx))];
  }
}

// NVFP4 metadata per expert: the E4M3 region (e4m3_src_index), then the fp32
// tensor scale of that expert and 12 zero bytes.
__global__ void repack_nvfp4_meta_kernel(const uint8_t* __restrict__ e4, const float* __restrict__ tscale,
                                         uint8_t* __restrict__ out, int64_t K, int64_t per, int64_t mpe,
                                         int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / mpe;
    const int64_t idx = i - e * mpe;
    uint8_t v = 0;
    if (idx < per) v = e4[e * per + e4m3_src_index(K, idx)];
    else if (idx < per + 4) v = reinterpret_cast<const uint8_t*>(tscale + e)[idx - per];
    out[i] = v;
  }
}

static dim3 grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return dim3((unsigned)b);
}

int launch_repack(const hq_plan* p, const void* codes, const void* scales, const void* zx, void* w_out,
                  void* meta_out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t N = p->layer.n, K = p->layer.k, E = p->layer.num_experts;
  const int64_t G = K / kFragK;
  if (w3_weights(p->fmt)) {
    const int64_t wpe3 = N * K * 3 / 32;  // 32-bit words per expert (same count as canonical)
    hipLaunchKernelGGL(repack_codes3_kernel, grid_for(wpe3 * E), dim3(256), 0, s, static_cast<const uint32_t*>(codes),
                       static_cast<uint32_t*>(w_out), K, wpe3, wpe3 * E);
  } else if (w2_weights(p->fmt)) {
    const int64_t wpe2 = N * K / 16;  // 32-bit words per expert (same count as canonical)
    hipLaunchKernelGGL(repack_codes2_kernel, grid_for(wpe2 * E), dim3(256), 0, s, static_cast<const uint32_t*>(codes),
                       static_cast<uint32_t*>(w_out), K, wpe2, wpe2 * E);
  } else if (w8_weights(p->fmt)) {
    const int64_t wpe8 = N * K / 4;  // 32-bit words per expert (one byte per weight)
    hipLaunchKernelGGL(repack_codes8_kernel, grid_for(wpe8 * E), dim3(256), 0, s, static_cast<const uint8_t*>(codes),
                       static_cast<uint32_t*>(w_out), K, wpe8, wpe8 * E);
  } else {
    const int64_t wpe = N * K / 8;  // 32-bit words per expert (same count as canonical)
    hipLaunchKernelGGL(repack_codes_kernel, grid_for(wpe * E), dim3(256), 0, s,
                       static_cast<const uint32_t*>(codes), static_cast<uint32_t*>(w_out), K, p->fmt, wpe,
                       wpe * E, wpe);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return (int)err;
  uint8_t* meta = static_cast<uint8_t*>(meta_out);
  const size_t mpe = p->meta_bytes_per_expert;
  if (nvfp4_weights(p->fmt)) {
    const int64_t per = N * K / 16;
    const int64_t mpe = (int64_t)p->meta_bytes_per_expert;
    hipLaunchKernelGGL(repack_nvfp4_meta_kernel, grid_for(mpe * E), dim3(256), 0, s, static_cast<const uint8_t*>(zx),
                       static_cast<const float*>(scales), meta, K, per, mpe, mpe * E);
    return (int)hipGetLastError();
  }
  if (e8m0_meta(p->fmt)) {
    // per expert: E8M0 region only (MXINT4: one dword of four block scales per column)
    const int64_t per = N * K / 32;
    hipLaunchKernelGGL(repack_e8m0_kernel, grid_for(per * E), dim3(256), 0, s,
                       static_cast<const uint8_t*>(zx), meta, K, per, per * E, mxint4_weights(p->fmt) ? 1 : 0);
    return (int)hipGetLastError();
  }
  // scales of every expert first, then zero points of every expert
  const int64_t sper = N * G;
  hipLaunchKernelGGL(repack_scales_kernel, grid_for(sper * E), dim3(256), 0, s,
                     static_cast<const uint16_t*>(scales), reinterpret_cast<uint16_t*>(meta), G, sper,
                     sper * E);
  err = hipGetLastError();
  if (err != hipSuccess) return (int)err;
  if (p->layer.q.zp == HQ_ZP_PER_GROUP_U4) {
    const int64_t zwpe = (N / 16) * G * 2;
    hipLaunchKernelGGL(repack_zeros_kernel, grid_for(zwpe * E), dim3(256), 0, s,
                       static_cast<const uint8_t*>(zx),
                       reinterpret_cast<uint32_t*>(meta + p->scale_region_bytes * E), G, zwpe, N * G,
                       zwpe * E);
    err = hipGetLastError();
  }
  (void)mpe;
  return (int)err;
}

}  // namespace hq
