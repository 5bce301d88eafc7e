// Per-token (per-row) activation quantiser: the step that produces the 8-bit
// activations and per-row fp32 scales a W4A8 GEMM consumes.
//
// The pages name W4A8 (4-bit weights, 8-bit activations: INT8 or FP8, with
// MXFP4 weights taking FP8 activations) but not how the activations are
// quantised (Humming page on news.ditty.ir, summary; cocoloop.cn, format
// section).  The rule here is the plainest symmetric per-row form:
//   s[m]      = max_k |x[m,k]| / Q   (fp32; s = 1 for an all-zero row)
//   code[m,k] = RNE(x[m,k] / s[m])   (correctly rounded fp32 quotient,
//                                     saturated to +-Q)
// with Q = 448 and an OCP e4m3fn code for FP8 (a negative value that rounds
// to zero gives code 0), Q = 127 and a two's-complement byte for INT8, so
// that code * s[m] approximates x[m,k].  The fused requantisation of the MoE
// gate_up output (moe.hip) follows the same rule.
//
// Layout: x [m, k] fp16/bf16 row-major, codes [m, k] bytes, scales [m] fp32.
// One workgroup per row: every thread loads its 16-byte chunks of the row
// into registers (all loads in flight at once), the row maximum is reduced
// across the workgroup, and the same registers are quantised and stored as
// 8-byte chunks.  Rows longer than the register cache (8 chunks per thread)
// read the rest twice; the second read hits the L2 this workgroup filled.
// With few rows a workgroup has up to 16 waves, so that the per-row chain
// (load, reduce, convert) is spread over more lanes; with many rows, 4 waves
// keep every row of a launch resident at once.  The e4m3 rounding is the
// hardware conversion (round to nearest even on the OCP format, input
// clamped to +-448 first).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "hq_internal.h"
#include "launch.h"

namespace hq {

namespace {

constexpr int kCache = 8;  // 16-byte chunks per thread held in registers

template <bool BF16>
__device__ inline float elem(uint32_t w, int hi) {
  const uint32_t b = hi ? (w >> 16) : (w & 0xFFFFu);
  return BF16 ? bf16_bits_to_float(b) : f16_bits_to_float(b);
}

template <bool BF16>
__device__ inline float chunk_absmax(u4_t v) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(elem<BF16>(v[j >> 1], j & 1)));
  return m;
}

// Eight quantised bytes of one chunk, little-endian in two words.  The
// quotient is the correctly rounded fp32 division (hipcc's default for '/').
template <bool BF16, bool FP8>
__device__ inline uint2 chunk_codes(u4_t v, float s) {
  float f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = elem<BF16>(v[j >> 1], j & 1) / s;
  uint32_t w[2];
  if constexpr (FP8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* g = f + 4 * h;
      int t = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(g[0], 448.f, -448.f),
                                              __builtin_amdgcn_fmed3f(g[1], 448.f, -448.f), 0, false);
      t = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(g[2], 448.f, -448.f),
                                          __builtin_amdgcn_fmed3f(g[3], 448.f, -448.f), t, true);
      // -0 (sign bit over a zero magnitude) -> 0: keep a byte's sign bit only
      // where its low seven bits are not all zero
      const uint32_t u = (uint32_t)t;
      const uint32_t nz = ((u & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;
      w[h] = u & (0x7F7F7F7Fu | nz);
    }
  } else {
    w[0] = w[1] = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(f[j]), 127.f, -127.f);
      w[j >> 2] |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * (j & 3));
    }
  }
  return uint2{w[0], w[1]};
}

template <bool BF16, bool FP8>
__global__ void __launch_bounds__(1024) quantize_rows_kernel(const u4_t* __restrict__ x, int64_t k8,
                                                             uint2* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float wmax[16];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  const u4_t* xr = x + row * k8;
  uint2* cr = codes + row * k8;

  u4_t v[kCache];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kCache; ++i) {
    const int64_t c = tid + (int64_t)i * nt;
    v[i] = c < k8 ? __builtin_nontemporal_load(xr + c) : u4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < kCache; ++i) amax = fmaxf(amax, chunk_absmax<BF16>(v[i]));
  for (int64_t c = tid + (int64_t)kCache * nt; c < k8; c += nt) amax = fmaxf(amax, chunk_absmax<BF16>(xr[c]));

  // row maximum: within the wave, then across the (up to 16) waves
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
  for (int w = 1; w < (nt >> 6); ++w) amax = fmaxf(amax, wmax[w]);

  const float s = amax > 0.f ? amax / (FP8 ? 448.f : 127.f) : 1.f;
#pragma unroll
  for (int i = 0; i < kCache; ++i) {
    const int64_t c = tid + (int64_t)i * nt;
    if (c < k8) cr[c] = chunk_codes<BF16, FP8>(v[i], s);
  }
  for (int64_t c = tid + (int64_t)kCache * nt; c < k8; c += nt) cr[c] = chunk_codes<BF16, FP8>(xr[c], s);
  if (tid == 0) scales[row] = s;
}

// ---------------------------------------------------------------------------
// MXFP4 block quantiser (activations of W4A4), after the OCP MX v1.0
// conversion of a 32-element block: shared exponent X = floor(log2 max|v|) - 2
// (2 = the largest E2M1 exponent), clamped to [-127, 127], X = 0 for an
// all-zero block; elements RNE_E2M1(v / 2^X) saturated to +-6.  The scaling by
// 2^-X is exact (ldexp), so every decision is an exact comparison.

// Round-to-nearest-even fp32 -> E2M1 code, saturating at 6; -0 gives code 0.
// Below 1 the spacing is 0.5 (code = rint(2|x|)); above, the 23-bit mantissa
// is rounded to 1 bit (a carry moves into the exponent field).
__device__ inline uint32_t e2m1_code_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  const float a = fminf(fabsf(x), 6.f);
  uint32_t code;
  if (a < 1.f) {
    code = (uint32_t)__builtin_rintf(a * 2.f);
  } else {
    const uint32_t bits = __float_as_uint(a);
    const uint32_t e = (bits >> 23) - 127u + 1u;  // exponent field, bias 1
    const uint32_t mant = bits & 0x7FFFFFu;
    const uint32_t r = (mant + 0x1FFFFFu + ((mant >> 22) & 1u)) >> 22;  // 0..2
    code = (e << 1) + r;
  }
  return code == 0 ? 0u : (sign | code);
}

// One thread per 32-element block: 64 input bytes in, 16 code bytes and one
// E8M0 byte out (consecutive threads, consecutive blocks of a row).  The
// scales are stored group-major: byte j of word (g, row) is block 4 g + j of
// the row, so that the GEMM's 16 rows of one operand read 64 contiguous bytes.
template <bool BF16>
__global__ void __launch_bounds__(256) quantize_mx_kernel(const u4_t* __restrict__ x, int64_t nblk, int64_t m,
                                                          int64_t kb, u4_t* __restrict__ codes,
                                                          uint8_t* __restrict__ e8m0) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblk) return;
  const int64_t row = i / kb, b = i - row * kb;
  u4_t v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = __builtin_nontemporal_load(x + 4 * i + c);
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) amax = fmaxf(amax, chunk_absmax<BF16>(v[c]));
  // floor(log2 amax) from the exponent field (a subnormal amax clamps to -127)
  const int X = amax > 0.f ? max((int)(__float_as_uint(amax) >> 23) - 127 - 2, -127) : 0;
  uint32_t w[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {  // chunk c: elements 8c .. 8c + 7 -> word c, low nibble first
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      word |= e2m1_code_rne(__builtin_amdgcn_ldexpf(elem<BF16>(v[c][j >> 1], j & 1), -X)) << (4 * j);
    w[c] = word;
  }
  codes[i] = u4_t{w[0], w[1], w[2], w[3]};
  e8m0[((b >> 2) * m + row) * 4 + (b & 3)] = (uint8_t)(X + 127);
}

}  // namespace

int launch_quantize_mx(int64_t m, int64_t k, int in_bf16, const void* x, void* codes, uint8_t* e8m0, void* stream) {
  const int64_t nblk = m * (k / 32);
  const dim3 grid((unsigned)((nblk + 255) / 256)), block(256);
  const auto xs = static_cast<const u4_t*>(x);
  const auto cs = static_cast<u4_t*>(codes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t kb = k / 32;
  return in_bf16 ? (int)launch_timed(quantize_mx_kernel<true>, grid, block, 0, s, xs, nblk, m, kb, cs, e8m0)
                 : (int)launch_timed(quantize_mx_kernel<false>, grid, block, 0, s, xs, nblk, m, kb, cs, e8m0);
}

int launch_quantize_rows(int64_t m, int64_t k, int in_bf16, int out_fp8, const void* x, void* codes, float* scales,
                         void* stream) {
  const int64_t k8 = k / 8;
  // one wave per 64 chunks of the row, at most 16 waves for up to 256 rows
  // and 4 waves beyond (every row of the launch then fits on the chip at once)
  const int64_t max_threads = m <= 256 ? 1024 : 256;
  const int threads = (int)std::min<int64_t>(max_threads, (k8 + 63) / 64 * 64);
  const auto xs = static_cast<const u4_t*>(x);
  const auto cs = static_cast<uint2*>(codes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)m), block((unsigned)threads);
  if (in_bf16)
    return out_fp8 ? (int)launch_timed(quantize_rows_kernel<true, true>, grid, block, 0, s, xs, k8, cs, scales)
                   : (int)launch_timed(quantize_rows_kernel<true, false>, grid, block, 0, s, xs, k8, cs, scales);
  return out_fp8 ? (int)launch_timed(quantize_rows_kernel<false, true>, grid, block, 0, s, xs, k8, cs, scales)
                 : (int)launch_timed(quantize_rows_kernel<false, false>, grid, block, 0, s, xs, k8, cs, scales);
}

}  // namespace hq
