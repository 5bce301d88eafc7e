// Mixture-of-experts helpers around the grouped GEMM: the token sort / align
// by expert, the per-row fp8 requantisation of the gate_up activation, and
// the top-k combine of the down projection's weighted slot rows.
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
// Slot ids outside [0, E) go to one trailing segment (pseudo-expert E) whose
// blocks are marked block_expert = -1: the GEMMs give those slots no output
// (gate_up) or a zero row (down), so they add nothing to the combine.
__global__ void __launch_bounds__(1024) moe_align_kernel(const int32_t* __restrict__ ids, int n_slots, int E,
                                                         int bm, int32_t* __restrict__ sorted_ids,
                                                         int32_t* __restrict__ block_expert,
                                                         int32_t* __restrict__ num_padded) {
  extern __shared__ int sh[];
  const int S = E + 1;         // segments: the experts, then the out-of-range slots
  int* cnt = sh;               // [S]
  int* off = sh + S;           // [S + 1] padded segment starts
  int* cur = sh + 2 * S + 1;   // [S] scatter cursors
  const int tid = threadIdx.x;
  for (int e = tid; e < S; e += blockDim.x) {
    cnt[e] = 0;
    cur[e] = 0;
  }
  __syncthreads();
  // ids are read in batches of kBatch per thread, all loads of a batch in
  // flight before its LDS atomics (one load per iteration would wait a full
  // memory latency per id)
  constexpr int kBatch = 8;
  const int nt = blockDim.x;
  for (int base = tid; base < n_slots; base += kBatch * nt) {
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) ev[u] = base + u * nt < n_slots ? ids[base + u * nt] : 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (base + u * nt < n_slots) atomicAdd(&cnt[(ev[u] >= 0 && ev[u] < E) ? ev[u] : E], 1);
  }
  __syncthreads();
  // padded sizes, then an inclusive scan over the segments by the first wave
  // (each lane owns a contiguous run of segments)
  if (tid < 64) {
    const int per = (S + 63) / 64;
    const int b0 = tid * per, b1 = min(S, b0 + per);
    int run = 0;
    for (int e = b0; e < b1; ++e) run += (cnt[e] + bm - 1) / bm * bm;
    int incl = run;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (tid >= d) incl += o;
    }
    int acc = incl - run;  // exclusive start of this lane's run
    for (int e = b0; e < b1; ++e) {
      off[e] = acc;
      acc += (cnt[e] + bm - 1) / bm * bm;
    }
    if (tid == 63) {
      off[S] = incl;
      *num_padded = incl;
    }
  }
  __syncthreads();
  const int total = off[S];
  for (int i = tid; i < total; i += blockDim.x) sorted_ids[i] = n_slots;
  for (int b = tid; b < total / bm; b += blockDim.x) {
    // the segment that contains row b * bm
    int lo = 0, hi = S;  // off[lo] <= b*bm < off[hi]
    const int row = b * bm;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= row) lo = mid;
      else hi = mid;
    }
    block_expert[b] = lo < E ? lo : -1;
  }
  __syncthreads();  // sentinel fill (global) before the scatter in this workgroup
  for (int base = tid; base < n_slots; base += kBatch * nt) {
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) ev[u] = base + u * nt < n_slots ? ids[base + u * nt] : 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (base + u * nt >= n_slots) continue;
      const int e = (ev[u] >= 0 && ev[u] < E) ? ev[u] : E;
      const int pos = off[e] + atomicAdd(&cur[e], 1);
      sorted_ids[pos] = base + u * nt;
    }
  }
}

// One wave per aligned row of the fp32 activations the gate_up epilogue
// stored: s = max|act| / 448 (1 for an all-zero row), codes = RNE_e4m3(act /
// s) with a correctly rounded fp32 quotient, saturated to +-448 -- the rule of
// the standalone per-token quantiser (quantize.hip).  The row maximum is
// formed here from the stored row (two passes over 4 * inter bytes, the
// second from the cache), so no state carries over between calls.  Rows are
// aligned positions (padding skipped), or slots when sorted_ids and
// num_padded are null.
__global__ void __launch_bounds__(256) moe_requant_kernel(const float* __restrict__ act32,
                                                          const int32_t* __restrict__ sorted_ids,
                                                          const int32_t* __restrict__ num_padded, int n_slots,
                                                          int inter, int64_t max_rows, uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= max_rows || (num_padded && row >= *num_padded)) return;
  if (sorted_ids && sorted_ids[row] >= n_slots) return;
  // four consecutive values per lane and access (inter is a multiple of 4)
  const float4* a = reinterpret_cast<const float4*>(act32 + row * inter);
  uint32_t* q = reinterpret_cast<uint32_t*>(codes + row * inter);
  const int n4 = inter >> 2;
  float amax = 0.f;
  for (int c = lane; c < n4; c += 64) {
    const float4 v = a[c];
    amax = fmaxf(fmaxf(amax, fabsf(v.x)), fmaxf(fmaxf(fabsf(v.y), fabsf(v.z)), fabsf(v.w)));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  const float s = amax > 0.f ? amax / 448.f : 1.f;
  for (int c = lane; c < n4; c += 64) {
    const float4 v = a[c];
    q[c] = e4m3_code_rne(v.x / s) | (e4m3_code_rne(v.y / s) << 8) | (e4m3_code_rne(v.z / s) << 16) |
           (e4m3_code_rne(v.w / s) << 24);
  }
  if (lane == 0) scales[row] = s;
}

// The combine: y[t, col0 + c] = RNE(sum_j rows[t * topk + j][c]) over the
// token's topk slot rows (each already weighted and rounded to bf16; rows of
// ncol columns, the down GEMM's column window), summed in fp32 in slot order;
// four outputs per thread (ncol and col0 are multiples of 4).
__global__ void __launch_bounds__(256) moe_combine_kernel(const uint2* __restrict__ rows, int topk, int64_t n4,
                                                          int64_t col04, int64_t ncol4, int64_t elems4,
                                                          uint2* __restrict__ y, int out_bf16) {
  auto lo = [](uint32_t b) { return __uint_as_float(b << 16); };
  auto hi = [](uint32_t b) { return __uint_as_float(b & 0xFFFF0000u); };
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < elems4; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / ncol4, c = i - t * ncol4;
    const uint2* r = rows + t * topk * ncol4 + c;
    const uint2 w0 = r[0];
    float4 v = make_float4(lo(w0.x), hi(w0.x), lo(w0.y), hi(w0.y));
    for (int j = 1; j < topk; ++j) {
      const uint2 w = r[(int64_t)j * ncol4];
      v.x += lo(w.x);
      v.y += hi(w.x);
      v.z += lo(w.y);
      v.w += hi(w.y);
    }
    const uint32_t h0 = out_bf16 ? float_to_bf16_bits(v.x) : float_to_f16_bits(v.x);
    const uint32_t h1 = out_bf16 ? float_to_bf16_bits(v.y) : float_to_f16_bits(v.y);
    const uint32_t h2 = out_bf16 ? float_to_bf16_bits(v.z) : float_to_f16_bits(v.z);
    const uint32_t h3 = out_bf16 ? float_to_bf16_bits(v.w) : float_to_f16_bits(v.w);
    y[t * n4 + col04 + c] = uint2{h0 | (h1 << 16), h2 | (h3 << 16)};
  }
}

int launch_moe_align(int64_t t, int topk, int num_experts, int block_m, const int32_t* ids, int32_t* sorted_ids,
                     int32_t* block_expert, int32_t* num_padded, void* stream) {
  const size_t lds = (size_t)(3 * (num_experts + 1) + 1) * sizeof(int);
  return (int)launch_timed(moe_align_kernel, dim3(1), dim3(1024), lds, static_cast<hipStream_t>(stream), ids,
                           (int)(t * topk), num_experts, block_m, sorted_ids, block_expert, num_padded);
}

int launch_moe_requant(const float* act32, const int32_t* sorted_ids, const int32_t* num_padded, int n_slots,
                       int inter, int64_t max_rows, uint8_t* codes, float* scales, void* stream) {
  if (inter % 4 || max_rows < 1) return (int)hipErrorInvalidValue;
  const int64_t blocks = (max_rows + 3) / 4;
  return (int)launch_timed(moe_requant_kernel, dim3((unsigned)blocks), dim3(256), 0,
                           static_cast<hipStream_t>(stream), act32, sorted_ids, num_padded, n_slots, inter, max_rows,
                           codes, scales);
}

int launch_moe_combine(const uint16_t* rows, int topk, int64_t t, int64_t n, int64_t col0, int64_t ncol, void* y,
                       int out_bf16, void* stream) {
  if (n % 4 || col0 % 4 || ncol % 4 || col0 < 0 || col0 + ncol > n) return (int)hipErrorInvalidValue;
  const int64_t elems4 = t * ncol / 4;
  int64_t blocks = (elems4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return (int)launch_timed(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                           reinterpret_cast<const uint2*>(rows), topk, n / 4, col0 / 4, ncol / 4, elems4,
                           static_cast<uint2*>(y), out_bf16);
}

}  // namespace hq
