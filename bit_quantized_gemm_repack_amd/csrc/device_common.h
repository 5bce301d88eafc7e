// Device helpers shared by the gfx950 GEMM kernels: operand vector types,
// 16-bit conversions, and the 4-bit code -> MFMA operand expansions that the
// fragment layout (hq_internal.h) was designed for.
#pragma once

#ifndef __HIPCC_RTC__  // the run-time compiler includes the HIP runtime itself
#include <hip/hip_runtime.h>
#endif

#include <cstdint>

namespace hq {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));
typedef int i8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ inline float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }
__device__ inline float f16_bits_to_float(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }

// Round-to-nearest-even fp32 -> bf16 bits: the hardware conversion (one
// v_cvt_pk_bf16_f32 on gfx950, round to nearest even, a NaN gives a quiet NaN).
__device__ inline uint16_t float_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Round-to-nearest-even fp32 -> fp16 bits (the hardware conversion).
__device__ inline uint16_t float_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Round-to-nearest-even fp32 -> OCP e4m3 (fn) code, saturating at 448; -0
// gives code 0.  Below 2^-5 the subnormal and first normal binade share the
// spacing 2^-9, so the code is the integer rint(|x| * 2^9); above it the
// 23-bit mantissa is rounded to 3 bits (a carry moves into the exponent).
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

__device__ inline i8_t cat8(u4_t x, u4_t y) {
  i8_t r;
  r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
  r[4] = y[0]; r[5] = y[1]; r[6] = y[2]; r[7] = y[3];
  return r;
}

// LDS address operand of the direct global->LDS buffer loads.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// A value the compiler cannot see through (kept in a VGPR).  Passing the
// magic exponent of w16_operand this way lets each register be one
// v_and_or_b32 (mask from an SGPR, magic from a VGPR): with both constants
// literal the compiler emits a separate AND and OR, as one VOP3 instruction
// cannot hold two literals.
__device__ inline uint32_t opaque_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// One word of NIB_W16 codes -> the 16-bit operand (8 values, k-offsets 0..7)
// holding MAGIC + q exactly: fp16 0x6400 = 1024, bf16 0x4300 = 128.
__device__ inline u4_t w16_operand(uint32_t x, uint32_t magic) {
  return u4_t{(x & 0x000F000Fu) | magic, ((x >> 4) & 0x000F000Fu) | magic, ((x >> 8) & 0x000F000Fu) | magic,
              ((x >> 12) & 0x000F000Fu) | magic};
}

// One word of INT2 codes -> the 16-bit operand of MFMA step 2d + u (the word
// holds steps 2d and 2d+1): register r = crumbs 4u + r (low half) and
// 8 + 4u + r (high half), MAGIC + q exactly.
__device__ inline u4_t w2_operand(uint32_t x, uint32_t magic, int u) {
  const uint32_t y = x >> (8 * u);
  return u4_t{(y & 0x00030003u) | magic, ((y >> 2) & 0x00030003u) | magic, ((y >> 4) & 0x00030003u) | magic,
              ((y >> 6) & 0x00030003u) | magic};
}

// One word of INT3 high bits -> the 16-bit operand of MFMA step t: register r
// = bits 4t + r (low half) and 16 + 4t + r (high half), MAGIC + bit exactly.
__device__ inline u4_t w1_operand(uint32_t x, uint32_t magic, int t) {
  const uint32_t y = x >> (4 * t);
  return u4_t{(y & 0x00010001u) | magic, ((y >> 1) & 0x00010001u) | magic, ((y >> 2) & 0x00010001u) | magic,
              ((y >> 3) & 0x00010001u) | magic};
}

// NVFP4 weights -> the 16-bit operand of one MFMA step, dequantised exactly.
// x holds the step's 8 E2M1 codes in the 16-bit operand order (nibbles r and
// 4 + r are elements 2r and 2r + 1); sb is the E4M3 code of their 16-k block.
// Each value is e2m1(q) * e4m3(sb) * 2^-8: the E2M1 bits placed as an fp16
// (sign to bit 15, exponent and mantissa to bits 9..11) are e2m1(q) * 2^-14;
// the E4M3 bits placed as an fp16 are e4m3(sb) * 2^-8, times 2^14 exactly;
// their product has at most 6 significant bits and lies in [2^-18, 10.5], so
// it is exact in fp16 and, widened and truncated, in bf16.  The kernel's
// epilogue multiplies by 2^8 and the tensor scale.  An E4M3 NaN code gives NaN.
template <bool BF16>
__device__ inline u4_t nvfp4_operand(uint32_t x, uint32_t sb) {
  _Float16 S = __builtin_bit_cast(_Float16, (uint16_t)(((sb & 0x80u) << 8) | ((sb & 0x7Fu) << 7))) * (_Float16)16384.f;
  if ((sb & 0x7Fu) == 0x7Fu) S = (_Float16)__builtin_nanf("");
  const h2_t S2 = h2_t{S, S};
  u4_t out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t u = (x >> (4 * r)) & 0x000F000Fu;
    const uint32_t bits = ((u & 0x00070007u) << 9) | ((u & 0x00080008u) << 12);
    const h2_t v = __builtin_bit_cast(h2_t, bits) * S2;
    if constexpr (BF16) {
      const uint32_t lo = __builtin_bit_cast(uint32_t, (float)v[0]);
      const uint32_t hi = __builtin_bit_cast(uint32_t, (float)v[1]);
      out[r] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // the upper halves: exact bf16
    } else {
      out[r] = __builtin_bit_cast(uint32_t, v);
    }
  }
  return out;
}

// Two words of NIB_B8 codes stored as q ^ 8 -> the int8 operand (16 values)
// holding 16 * (q - 8) exactly.
__device__ inline i4_t i8_operand(uint32_t w0, uint32_t w1) {
  return i4_t{(int)((w0 << 4) & 0xF0F0F0F0u), (int)(w0 & 0xF0F0F0F0u), (int)((w1 << 4) & 0xF0F0F0F0u),
              (int)(w1 & 0xF0F0F0F0u)};
}

// Four words of NIB_B8 codes -> the fp8 operand (32 values): the e4m3 codes
// 0x00..0x0F, i.e. q * 2^-9 exactly (subnormal and first normal binade share
// the spacing 2^-9).
__device__ inline i8_t q8_operand(u4_t w) {
  return i8_t{(int)(w[0] & 0x0F0F0F0Fu), (int)((w[0] >> 4) & 0x0F0F0F0Fu), (int)(w[1] & 0x0F0F0F0Fu),
              (int)((w[1] >> 4) & 0x0F0F0F0Fu), (int)(w[2] & 0x0F0F0F0Fu), (int)((w[2] >> 4) & 0x0F0F0F0Fu),
              (int)(w[3] & 0x0F0F0F0Fu), (int)((w[3] >> 4) & 0x0F0F0F0Fu)};
}

template <bool F16>
__device__ inline f4_t mfma_16x16x32(u4_t a, u4_t b, f4_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a), __builtin_bit_cast(b8_t, b), c,
                                                   0, 0, 0);
}

__device__ inline float load_scale(const void* scales, int64_t idx, int bf16) {
  const uint32_t s = static_cast<const uint16_t*>(scales)[idx];
  return bf16 ? bf16_bits_to_float(s) : f16_bits_to_float(s);
}

__device__ inline void store_out(void* out, int64_t idx, float v, int bf16) {
  static_cast<uint16_t*>(out)[idx] = bf16 ? float_to_bf16_bits(v) : float_to_f16_bits(v);
}

}  // namespace hq
