// Mixture-of-experts helpers around the grouped GEMM: the token sort / align
// by expert, the per-row fp8 requantisation of the gate_up activation, and
// the final fp32 -> bf16/fp16 conversion of the combined down projection.
//
// The pages describe a dedicated MoE backend whose "Grouped" GEMM path is run
// with W4A16 or W4A8 weights (Humming page on news.ditty.ir, summary;
// cocoloop.cn speed-up table, MoE row).  They do not describe the routing
// data structures; the alignment below is the plainest form the grouped GEMM
// needs: every expert's slots contiguous and padded to whole row blocks.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "hq_internal.h"
#include "launch.h"

namespace hq {

// One workgroup: histogram of expert ids in LDS, padded exclusive prefix
// sum, sentinel fill, block -> expert table, then the scatter of slot ids.
// Slot ids outside [0, E) are ignored (left out of every segment).
__global__ void __launch_bounds__(1024) moe_align_kernel(const int32_t* __restrict__ ids, int n_slots, int E,
                                                         int bm, int32_t* __restrict__ sorted_ids,
                                                         int32_t* __restrict__ block_expert,
                                                         int32_t* __restrict__ num_padded) {
  extern __shared__ int sh[];
  int* cnt = sh;           // [E]
  int* off = sh + E;       // [E + 1] padded segment starts
  int* cur = sh + 2 * E + 1;  // [E] scatter cursors
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    cnt[e] = 0;
    cur[e] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n_slots; i += blockDim.x) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = acc;
      acc += (cnt[e] + bm - 1) / bm * bm;
    }
    off[E] = acc;
    *num_padded = acc;
  }
  __syncthreads();
  const int total = off[E];
  for (int i = tid; i < total; i += blockDim.x) sorted_ids[i] = n_slots;
  for (int b = tid; b < total / bm; b += blockDim.x) {
    // the expert whose padded segment contains row b * bm
    int lo = 0, hi = E;  // off[lo] <= b*bm < off[hi]
    const int row = b * bm;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= row) lo = mid;
      else hi = mid;
    }
    block_expert[b] = lo;
  }
  __syncthreads();  // sentinel fill (global) before the scatter in this workgroup
  for (int i = tid; i < n_slots; i += blockDim.x) {
    const int e = ids[i];
    if (e < 0 || e >= E) continue;
    const int pos = off[e] + atomicAdd(&cur[e], 1);
    sorted_ids[pos] = i;
  }
}

// Round-to-nearest-even fp32 -> OCP e4m3 code for |x| <= 448.  Below 2^-5 the
// subnormal and first normal binade share the spacing 2^-9, so the code is
// the integer rint(|x| * 2^9); above it the 23-bit mantissa is rounded to 3
// bits (a carry moves into the exponent field).
__device__ inline uint32_t e4m3_code_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  uint32_t code;
  if (a < 0.03125f) {
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const uint32_t bits = __float_as_uint(a);
    const uint32_t exp = (bits >> 23) - 127u + 7u;
    const uint32_t mant = bits & 0x7FFFFFu;
    const uint32_t r = (mant + 0x7FFFFu + ((mant >> 20) & 1u)) >> 20;  // 0..8
    code = (exp << 3) + r;
  }
  return code == 0 ? 0u : (sign | code);
}

// One wave per aligned row: s = max|act| / 448 (1 for an all-zero row),
// codes = RNE_e4m3(act / s).  Resets the row maximum for the next call.
__global__ void __launch_bounds__(256) moe_requant_kernel(const float* __restrict__ act32,
                                                          uint32_t* __restrict__ row_amax,
                                                          const int32_t* __restrict__ sorted_ids,
                                                          const int32_t* __restrict__ num_padded, int n_slots,
                                                          int inter, int64_t max_rows, uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= max_rows || row >= *num_padded) return;
  if (sorted_ids[row] >= n_slots) return;
  const float amax = __uint_as_float(row_amax[row]);
  const float s = amax > 0.f ? amax / 448.f : 1.f;
  for (int col = lane; col < inter; col += 64) {
    const float v = act32[row * inter + col] / s;
    codes[row * inter + col] = (uint8_t)e4m3_code_rne(v);
  }
  if (lane == 0) {
    scales[row] = s;
    row_amax[row] = 0u;
  }
}

// y = RNE(y32) in the output dtype, and y32 back to zero for the next call.
__global__ void __launch_bounds__(256) moe_finalize_kernel(float* __restrict__ y32, void* __restrict__ y,
                                                           int64_t elems, int out_bf16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < elems; i += (int64_t)gridDim.x * blockDim.x) {
    store_out(y, i, y32[i], out_bf16);
    y32[i] = 0.f;
  }
}

int launch_moe_align(int64_t t, int topk, int num_experts, int block_m, const int32_t* ids, int32_t* sorted_ids,
                     int32_t* block_expert, int32_t* num_padded, void* stream) {
  const size_t lds = (size_t)(3 * num_experts + 1) * sizeof(int);
  hipLaunchKernelGGL(moe_align_kernel, dim3(1), dim3(1024), lds, static_cast<hipStream_t>(stream), ids,
                     (int)(t * topk), num_experts, block_m, sorted_ids, block_expert, num_padded);
  return (int)hipGetLastError();
}

int launch_moe_requant(const float* act32, uint32_t* row_amax, const int32_t* sorted_ids, const int32_t* num_padded,
                       int n_slots, int inter, int64_t max_rows, uint8_t* codes, float* scales, void* stream) {
  const int64_t blocks = (max_rows + 3) / 4;
  return (int)launch_timed(moe_requant_kernel, dim3((unsigned)blocks), dim3(256), 0,
                           static_cast<hipStream_t>(stream), act32, row_amax, sorted_ids, num_padded, n_slots, inter,
                           max_rows, codes, scales);
}

int launch_moe_finalize(float* y32, void* y, int64_t elems, int out_bf16, void* stream) {
  int64_t blocks = (elems + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return (int)launch_timed(moe_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0,
                           static_cast<hipStream_t>(stream), y32, y, elems, out_bf16);
}

}  // namespace hq
