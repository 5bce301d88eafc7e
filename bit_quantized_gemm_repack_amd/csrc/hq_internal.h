// Internal definitions shared by the host library and the gfx950 kernels.
//
// Device weight layout ("fragment" layout)
// ----------------------------------------
// The weight [N, K] is cut into fragments of 16 columns (n) x 128 k.  One
// fragment is exactly what one wavefront consumes with a single 16-byte load
// per lane: 64 lanes x 16 B = 1 KiB = 16 x 128 4-bit codes.  Fragments are
// stored n-block major: fragment (nb, g) sits at byte ((nb * K/128) + g) * 1024,
// so one wave walking along K reads one contiguous stream.
//
// Lane l of a fragment holds column c = l % 16 and 32 of the fragment's 128 k,
// split in pieces so that, for every load instruction of the activation
// operand (which takes row m = l % 16 in lane l), the four lanes of one row
// read one contiguous 64-byte run:
//
//   NIB_W16  (fp16 / bf16 MFMA 16x16x32, 4 steps of 32 k): word t (8 codes)
//            holds k = 32 t + 8 kq + [0, 8), kq = l / 16; nibble p holds the
//            k-offset {0,2,4,6,1,3,5,7}[p], so (w >> 4r) & 0x000F000F puts the
//            codes of k-offsets 2r and 2r+1 in the two 16-bit halves.
//   NIB_B8   (8-bit operands: int8 MFMA 16x16x64, fp8 scaled MFMA): two
//            pieces of 16 k, piece h = k 64 h + 16 kq + [0, 16) in words 2h,
//            2h+1; byte b of word 2h+u holds k-offset 8u + b in its low nibble
//            and 8u + 4 + b in its high nibble, so w & 0x0F0F0F0F /
//            (w >> 4) & 0x0F0F0F0F (or the 0xF0F0F0F0 forms) give four
//            consecutive k as four bytes.
//   NIB_NAT  (MXFP4, fp4 operand of the scaled MFMA): the 32 consecutive k
//            [32 kq, 32 kq + 32) of the E8M0 block kq, nibble p of word t
//            holding k-offset 8 t + p (E2M1 operand order).  The fp8
//            activation operand of that instruction takes k 16 kq + [0, 16)
//            in registers 0-3 and 64 + 16 kq + [0, 16) in registers 4-7,
//            i.e. the same two pieces as NIB_B8.
//
// For the int8 MFMA the stored nibble is q ^ 8, the two's-complement int4 of
// q - 8: placed in the high half of a byte it reads as the int8 16 * (q - 8).
//
// Scales, zero points, E8M0: per (n-block, group) records in the order the
// lanes read them: scales [N/16][K/128][16] (2 B each), zero points as
// nibbles [N/16][K/128][16 x 4 bit] (8 B), E8M0 [N/16][K/128][64 lanes].
// A grouped (MoE) weight is E such layouts one after the other.
#pragma once

#include <cstdint>
#include <utility>
#ifndef __HIPCC_RTC__  // the run-time compiler sees the device-side definitions only
#include <cstddef>
#include <vector>

#include "../../include/hq.h"
#endif

#if defined(__HIPCC__)
#define HQ_HD __host__ __device__
#else
#define HQ_HD
#endif

namespace hq {

constexpr int kFragN = 16;
constexpr int kFragK = 128;
constexpr int kFragBytes = 1024;

// Kernel-side format of the weight x activation pair.
enum Fmt : int {
  FMT_W16F16 = 0,  // INT4 weight, fp16 activation, fp16 MFMA
  FMT_W16BF16 = 1, // INT4 weight, bf16 activation, bf16 MFMA
  FMT_I8 = 2,      // INT4 weight, int8 activation, int8 MFMA (exact int32)
  FMT_Q8 = 3,      // INT4 weight, fp8 activation, scaled fp8 MFMA
  FMT_F4 = 4,      // MXFP4 weight, fp8 activation, scaled fp8 x fp4 MFMA
  FMT_F44 = 5,     // MXFP4 weight, MXFP4 activation, scaled fp4 x fp4 MFMA
  FMT_W8F16 = 6,   // INT8 weight, fp16 activation (two 4-bit planes), fp16 MFMA
  FMT_W8BF16 = 7,  // INT8 weight, bf16 activation (two 4-bit planes), bf16 MFMA
  FMT_W2F16 = 8,   // INT2 weight, fp16 activation, fp16 MFMA
  FMT_W2BF16 = 9,  // INT2 weight, bf16 activation, bf16 MFMA
  FMT_W3F16 = 10,  // INT3 weight, fp16 activation (2-bit + 1-bit planes), fp16 MFMA
  FMT_W3BF16 = 11, // INT3 weight, bf16 activation (2-bit + 1-bit planes), bf16 MFMA
  FMT_MX4F16 = 12, // MXINT4 weight (E8M0 per 32 k), fp16 activation, fp16 MFMA
  FMT_MX4BF16 = 13, // MXINT4 weight (E8M0 per 32 k), bf16 activation, bf16 MFMA
  FMT_NV4F16 = 14,  // NVFP4 weight (E4M3 per 16 k + fp32 tensor scale), fp16 activation, fp16 MFMA
  FMT_NV4BF16 = 15  // NVFP4 weight, bf16 activation, bf16 MFMA
};

// INT8 weights: stored as two 4-bit planes (high nibbles, then low nibbles)
// in the 16-bit operand order, so that each plane expands to exact MFMA
// operands like an INT4 weight and q = 16 * high + low.
HQ_HD constexpr inline bool w8_weights(int fmt) { return fmt == FMT_W8F16 || fmt == FMT_W8BF16; }
// INT2 weights: 512-byte fragments, 8 bytes per lane, 16 codes per word.
HQ_HD constexpr inline bool w2_weights(int fmt) { return fmt == FMT_W2F16 || fmt == FMT_W2BF16; }
// INT3 weights: 768-byte fragments, a 2-bit plane of the low code bits in the
// INT2 layout (512 bytes) then a 1-bit plane of the high bits (256 bytes, one
// word per lane), q = 4 * high + low.
HQ_HD constexpr inline bool w3_weights(int fmt) { return fmt == FMT_W3F16 || fmt == FMT_W3BF16; }
// MXINT4 weights: two's-complement codes stored offset by 8 (q xor 8) in the
// 16-bit operand order, one E8M0 scale per column per 32 k, i.e. per MFMA step.
HQ_HD constexpr inline bool mxint4_weights(int fmt) { return fmt == FMT_MX4F16 || fmt == FMT_MX4BF16; }
// NVFP4 weights: E2M1 codes in the 16-bit operand order, dequantised in
// registers (a lane's 8 k of one MFMA step lie in one 16-k block).
HQ_HD constexpr inline bool nvfp4_weights(int fmt) { return fmt == FMT_NV4F16 || fmt == FMT_NV4BF16; }
// fp16 / bf16 activations (INT2, INT3, INT4, INT8, MXINT4 or NVFP4 weights)
HQ_HD constexpr inline bool act16_fmt(int fmt) {
  return fmt == FMT_W16F16 || fmt == FMT_W16BF16 || fmt == FMT_W8F16 || fmt == FMT_W8BF16 || fmt == FMT_W2F16 ||
         fmt == FMT_W2BF16 || fmt == FMT_W3F16 || fmt == FMT_W3BF16 || fmt == FMT_MX4F16 || fmt == FMT_MX4BF16 ||
         fmt == FMT_NV4F16 || fmt == FMT_NV4BF16;
}
// fp16 (rather than bf16) activations
HQ_HD constexpr inline bool f16_act(int fmt) {
  return fmt == FMT_W16F16 || fmt == FMT_W8F16 || fmt == FMT_W2F16 || fmt == FMT_W3F16 || fmt == FMT_MX4F16 ||
         fmt == FMT_NV4F16;
}
// Weight bytes of one 16 x 128 fragment.
HQ_HD constexpr inline int frag_bytes(int fmt) {
  return w8_weights(fmt) ? 2048 : (w2_weights(fmt) ? 512 : (w3_weights(fmt) ? 768 : 1024));
}

// MXFP4 weights (E2M1 codes in natural order + E8M0 block scales).
HQ_HD constexpr inline bool mx_weights(int fmt) { return fmt == FMT_F4 || fmt == FMT_F44; }
// Metadata is one region of byte scales (E8M0 for MXFP4 / MXINT4, E4M3 for
// NVFP4) rather than 16-bit scales + zero points.
HQ_HD constexpr inline bool e8m0_meta(int fmt) { return mx_weights(fmt) || mxint4_weights(fmt) || nvfp4_weights(fmt); }
// Bytes of that region per 16 x 128 fragment.
HQ_HD constexpr inline int byte_meta_frag(int fmt) { return nvfp4_weights(fmt) ? 128 : 64; }

enum NibOrder : int { NIB_W16 = 0, NIB_B8 = 1, NIB_NAT = 2 };

HQ_HD inline int nib_order_of(int fmt) {
  return act16_fmt(fmt) ? NIB_W16 : (mx_weights(fmt) ? NIB_NAT : NIB_B8);
}
HQ_HD inline uint32_t nib_xor_of(int fmt) { return (fmt == FMT_I8 || mxint4_weights(fmt)) ? 8u : 0u; }

// k-offset (0..7, within the 8 k of one word) held by nibble p.
HQ_HD inline int nib_koff(int order, int p) {
  if (order == NIB_W16) return (p < 4) ? 2 * p : 2 * (p - 4) + 1;
  if (order == NIB_B8) return (p & 1) ? 4 + (p >> 1) : (p >> 1);
  return p;
}

// Canonical 4-bit code (n, k) of a row-major int32 [N, K/8] code matrix.
HQ_HD inline uint32_t canon_code(const uint32_t* codes, int64_t K, int64_t n, int64_t k) {
  return (codes[n * (K / 8) + (k >> 3)] >> (4 * (k & 7))) & 0xFu;
}

// First k (within the fragment's 128) of word t of the lane quarter kq.
HQ_HD inline int word_kbase(int order, int kq, int t) {
  if (order == NIB_W16) return 32 * t + 8 * kq;
  if (order == NIB_B8) return 64 * (t >> 1) + 16 * kq + 8 * (t & 1);
  return 32 * kq + 8 * t;
}

// One 32-bit word of the device layout: word index widx counts 32-bit words
// from the start of one expert's code region.
HQ_HD inline uint32_t repack_word(const uint32_t* codes, int64_t K, int fmt, int64_t widx) {
  const int64_t G = K / kFragK;
  const int t = (int)(widx & 3);
  const int lane = (int)((widx >> 2) & 63);
  const int64_t frag = widx >> 8;
  const int64_t g = frag % G;
  const int64_t nb = frag / G;
  const int64_t n = nb * kFragN + (lane & 15);
  const int order = nib_order_of(fmt);
  const int64_t kbase = g * kFragK + word_kbase(order, lane >> 4, t);
  const uint32_t x = nib_xor_of(fmt);
  uint32_t w = 0;
  for (int p = 0; p < 8; ++p) w |= (canon_code(codes, K, n, kbase + nib_koff(order, p)) ^ x) << (4 * p);
  return w;
}

// One 32-bit word of the INT8 device layout (two 1 KiB planes per 16 x 128
// fragment: high nibbles, then low nibbles, each in the 4-bit order of the
// 16-bit operands): word widx of one expert's region <- canonical uint8 [N][K].
HQ_HD inline uint32_t repack_word8(const uint8_t* codes, int64_t K, int64_t widx) {
  const int64_t G = K / kFragK;
  const int t = (int)(widx & 3);
  const int lane = (int)((widx >> 2) & 63);
  const int plane = (int)((widx >> 8) & 1);
  const int64_t frag = widx >> 9;
  const int64_t g = frag % G;
  const int64_t nb = frag / G;
  const int64_t n = nb * kFragN + (lane & 15);
  const int64_t kbase = g * kFragK + word_kbase(NIB_W16, lane >> 4, t);
  uint32_t w = 0;
  for (int p = 0; p < 8; ++p) {
    const uint32_t q = codes[n * K + kbase + nib_koff(NIB_W16, p)];
    w |= (plane == 0 ? (q >> 4) : (q & 0xFu)) << (4 * p);
  }
  return w;
}

// One 32-bit word of the INT2 device layout (512-byte fragments, two words
// per lane): word d of lane l holds the 16 codes of MFMA steps 2d and 2d+1;
// crumb 4u + r (u = 0, 1; r = 0..3) is element 2r of step 2d + u and crumb
// 8 + 4u + r element 2r + 1, so that (w >> 2(4u + r)) & 0x00030003 is operand
// register r of step 2d + u.  Canonical int32 [N][K/16], low bits first.
HQ_HD inline uint32_t repack_word2(const uint32_t* codes, int64_t K, int64_t widx) {
  const int64_t G = K / kFragK;
  const int d = (int)(widx & 1);
  const int lane = (int)((widx >> 1) & 63);
  const int64_t frag = widx >> 7;
  const int64_t g = frag % G;
  const int64_t nb = frag / G;
  const int64_t n = nb * kFragN + (lane & 15);
  uint32_t w = 0;
  for (int p = 0; p < 16; ++p) {
    const int hi = p >> 3, u = (p >> 2) & 1, r = p & 3;
    const int64_t k = g * kFragK + 32 * (2 * d + u) + 8 * (lane >> 4) + 2 * r + hi;
    const uint32_t q = (codes[n * (K / 16) + (k >> 4)] >> (2 * (k & 15))) & 0x3u;
    w |= q << (2 * p);
  }
  return w;
}

// Code k of one row of canonical INT3 words: the row is one little-endian bit
// stream and the code takes stream bits [3k, 3k+3) (it may straddle words).
HQ_HD inline uint32_t code3_at(const uint32_t* row, int64_t k) {
  const int64_t b = 3 * k;
  const int64_t j = b >> 5;
  const int o = (int)(b & 31);
  uint32_t v = row[j] >> o;
  if (o > 29) v |= row[j + 1] << (32 - o);
  return v & 0x7u;
}

// One 32-bit word of the INT3 device layout (768-byte fragments of 192
// words): words [0, 128) are the low two bits of every code in the INT2
// layout (repack_word2's crumb order), words [128, 192) the high bit, one word
// per lane: bit 4t + r is element 2r and bit 16 + 4t + r element 2r + 1 of
// MFMA step t, so that (w >> (4t + r)) & 0x00010001 is operand register r of
// step t.  Canonical int32 [N][3K/32], the dense 3-bit stream along K.
HQ_HD inline uint32_t repack_word3(const uint32_t* codes, int64_t K, int64_t widx) {
  const int64_t G = K / kFragK;
  const int64_t frag = widx / 192;
  const int rem = (int)(widx - frag * 192);
  const int64_t g = frag % G;
  const int64_t nb = frag / G;
  const bool high = rem >= 128;
  const int lane = high ? rem - 128 : rem >> 1;
  const int d = rem & 1;
  const int64_t n = nb * kFragN + (lane & 15);
  const uint32_t* row = codes + n * (K / 32 * 3);
  uint32_t w = 0;
  for (int p = 0; p < (high ? 32 : 16); ++p) {
    int64_t k;
    if (high) {
      const int hi = p >> 4, t = (p >> 2) & 3, r = p & 3;
      k = g * kFragK + 32 * t + 8 * (lane >> 4) + 2 * r + hi;
    } else {
      const int hi = p >> 3, u = (p >> 2) & 1, r = p & 3;
      k = g * kFragK + 32 * (2 * d + u) + 8 * (lane >> 4) + 2 * r + hi;
    }
    const uint32_t q = code3_at(row, k);
    w |= (high ? (q >> 2) : (q & 0x3u)) << (high ? p : 2 * p);
  }
  return w;
}

// Element eidx of the scale region [N/16][G][16] <- canonical [N][G].
HQ_HD inline int64_t scale_src_index(int64_t G, int64_t eidx) {
  const int64_t c = eidx & 15;
  const int64_t g = (eidx >> 4) % G;
  const int64_t nb = (eidx >> 4) / G;
  return (nb * kFragN + c) * G + g;
}

// 32-bit word widx of the zero-point region [N/16][G][2 words] (16 nibbles,
// column c at bits 4*(c%8) of word c/8) <- canonical uint8 [N][G].
HQ_HD inline uint32_t zeros_word(const uint8_t* zeros, int64_t G, int64_t widx) {
  const int half = (int)(widx & 1);
  const int64_t g = (widx >> 1) % G;
  const int64_t nb = (widx >> 1) / G;
  uint32_t w = 0;
  for (int i = 0; i < 8; ++i) {
    const int64_t n = nb * kFragN + half * 8 + i;
    w |= (uint32_t)(zeros[n * G + g] & 0xF) << (4 * i);
  }
  return w;
}

// Byte eidx of the E8M0 region [N/16][G][64 lanes] <- canonical [N][K/32].
HQ_HD inline int64_t e8m0_src_index(int64_t K, int64_t eidx) {
  const int64_t G = K / kFragK;
  const int lane = (int)(eidx & 63);
  const int64_t g = (eidx >> 6) % G;
  const int64_t nb = (eidx >> 6) / G;
  const int64_t n = nb * kFragN + (lane & 15);
  return n * (K / 32) + 4 * g + (lane >> 4);
}

// Byte eidx of the MXINT4 E8M0 region [N/16][G][16 columns][4 blocks] (one
// dword per column: the scales of its four MFMA steps) <- canonical [N][K/32].
HQ_HD inline int64_t e8m0_cols_src_index(int64_t K, int64_t eidx) {
  const int64_t G = K / kFragK;
  const int t = (int)(eidx & 3);
  const int c = (int)((eidx >> 2) & 15);
  const int64_t g = (eidx >> 6) % G;
  const int64_t nb = (eidx >> 6) / G;
  return (nb * kFragN + c) * (K / 32) + 4 * g + t;
}

// Byte eidx of the NVFP4 E4M3 region [N/16][G][16 columns][2 halves][4 steps]
// (lane (c, kq) reads the dword of half kq/2: byte t is the scale of the
// 16-k block 2t + kq/2 that its 8 k of MFMA step t fall in) <- canonical
// [N][K/16].
HQ_HD inline int64_t e4m3_src_index(int64_t K, int64_t eidx) {
  const int64_t G = K / kFragK;
  const int t = (int)(eidx & 3);
  const int h = (int)((eidx >> 2) & 1);
  const int c = (int)((eidx >> 3) & 15);
  const int64_t g = (eidx >> 7) % G;
  const int64_t nb = (eidx >> 7) / G;
  return (nb * kFragN + c) * (K / 16) + 8 * g + 2 * t + h;
}

// ---------------------------------------------------------------------------
// Plan
// ---------------------------------------------------------------------------

enum KernelKind : int { KER_SKINNY = 1, KER_TILED = 2 };

struct TiledCfgRt {
  int bm;     // rows per workgroup tile (64, 128)
  int nbw;    // 16-column blocks per wave (2, 4); tile width = 64 * nbw
  int split;   // K split over workgroups (dense; partials + reduce kernel)
  int stages;  // groups in the load pipeline (3; dense also 4, 5)
  int gm;      // launch order (dense): row tiles per group, the group's tiles column by column
};

struct SkinnyCfg {
  int mb;      // 16-row blocks per workgroup (1, 2, 4)
  int nb;      // 16-column blocks per workgroup (1, 2, 4)
  int waves;   // wavefronts per workgroup (split K inside the workgroup)
  int split;   // workgroups along K (1 = no cross-workgroup reduction)
  int stages;  // groups in flight per wave
};

}  // namespace hq

#ifndef __HIPCC_RTC__
struct hq_plan {
  hq_layer_desc layer;
  hq_compute compute;
  int64_t max_m;
  hq_tuning user;  // user overrides (zero = auto)
  // per-m execution choices installed by hq_plan_autotune / hq_plan_set_tuning
  // (dense plans); they take the place of `user` for exactly that m
  std::vector<std::pair<int64_t, hq_tuning>> tuned;
  int fmt;         // hq::Fmt
  size_t w_bytes_per_expert;
  size_t meta_bytes_per_expert;
  size_t scale_region_bytes;  // per expert, before the zero / e8m0 region
  int jit;                    // kernels specialised at run time for each call's shape (hq_plan_set_jit)
  char jit_dir[512];          // code-object cache directory ("" = the default)
};
#endif  // __HIPCC_RTC__

namespace hq {

#ifndef __HIPCC_RTC__
// Resolved execution choice for one call with m rows.
struct Exec {
  int kernel;
  SkinnyCfg sk;
  TiledCfgRt tl;
  int64_t tiles_m, tiles_n;
  size_t ws_bytes;  // total workspace: the fp32 split-K partials
};

// The execution choice for m rows: the heuristic with the overrides of `u`,
// or (u == nullptr) with the plan's tuned entry for m, else its user tuning.
Exec choose_exec(const hq_plan* p, int64_t m, const hq_tuning* u = nullptr);
#endif  // __HIPCC_RTC__

// Kernel arguments (passed by value) and launchers (defined in the .hip
// files; they return a hipError_t as int).
struct SkinnyArgs {
  const void* a;
  const float* a_scale;
  const uint8_t* a_e8m0;  // MXFP4 activations: E8M0 words [K/128][M][4]
  const void* w;
  const void* scales;
  const uint32_t* zeros;  // nibble-packed, or null
  const uint8_t* e8m0;
  const float* tscale;  // NVFP4: the fp32 tensor scale (device)
  void* out;
  float* part;       // [split][M][N] fp32 partials (split > 1)
  int M, N, K, G;
  int zp_fixed;      // fixed zero point, or -1 for per-group zeros
  int scale_bf16;    // scale dtype: 1 bf16, 0 fp16
  int out_bf16;      // output dtype: 1 bf16, 0 fp16
  int i32_out;       // write per-group int32 accumulators instead of C
  int gps;           // groups per split
  // ---- grouped (MoE) mode ----
  const int32_t* sorted_ids;    // aligned slot ids (sentinel n_slots)
  const int32_t* block_expert;  // expert of each aligned block
  const int32_t* num_padded;    // used length of sorted_ids
  const float* topk_w;          // [t, topk] routing weights (combine)
  int topk;
  int n_slots;                  // t * topk
  int epi;                      // EPI_* below
  int half_nblk;                // (n / 2) / 16: first up-projection column block
  int64_t w_expert;             // repacked code bytes per expert
  int64_t s_expert;             // scale elements per expert
  int64_t z_expert;             // zero-point words per expert
  int64_t e8_expert;            // E8M0 bytes per expert
  float* f32_out;               // gate_up fp32 act (QFP8)
  uint16_t* rows16;             // down: weighted slot rows, bf16 [n_slots][N] (small K: [n_slots][ncol])
  // small-K down GEMM: this launch covers columns [col0, col0 + ncol) of N
  // and stores slot rows [n_slots][ncol] (0, 0: all of N)
  int col0, ncol;
  // slot / token modes: the routing and the experts' layout
  const int32_t* topk_ids;  // [t][topk]
  int num_experts;
  int ge;                   // groups per expert (token mode: G = topk * ge)
  // dense 16-bit activations, one 16-row block per workgroup: bytes per row of
  // the workgroup's activation slab copied into LDS once (0: each wave loads
  // its groups' activations from global memory)
  int a_pitch;
};

// Grouped epilogues (SkinnyArgs::epi / TiledArgs::epi).
enum GroupedEpi : int { GEPI_PLAIN = 0, GEPI_SILU = 1, GEPI_SILU_F32 = 2, GEPI_COMBINE = 3 };
// Grouped kernel modes (template parameter): 0 dense, 1 rows gathered by
// token (gate_up), 2 rows in aligned order (down).
// 3 (skinny kernel, few tokens): block z is routed slot z, its expert read from
// topk_ids, its row token z / topk, gate_up output row z; 4 (skinny kernel,
// few tokens): block z is token z, the k loop walks its topk slots' rows and
// experts (groups g: slot g / ge, group g % ge), the top-k weight folded into
// each group's scale, so the workgroup's reduction is the combine.
enum GroupedMode : int { GRP_DENSE = 0, GRP_GATHER = 1, GRP_SORTED = 2, GRP_SLOT = 3, GRP_TOKEN = 4 };

#ifndef __HIPCC_RTC__
int launch_skinny(int fmt, const SkinnyCfg& cfg, const SkinnyArgs& a, void* stream);
// Grouped down GEMM for short K (K = 128 G): blocks of 16 mb aligned rows,
// combine rows out.  Supported: fp16 / bf16 / fp8 activations, mb 1 with
// G <= 4 (1, 2, 4), mb 4 with G <= 2.
bool smallk_supported(int fmt, int mb, int G);
int launch_smallk_grouped(int fmt, int mb, const SkinnyArgs& a, int64_t blocks, void* stream);
// Grouped launch: grid.z = blocks of the aligned array (max_padded / (16 mb)).
int launch_skinny_grouped(int fmt, int mode, const SkinnyCfg& cfg, const SkinnyArgs& a, int64_t blocks,
                          void* stream);
// Unaligned grouped launch (GRP_SLOT: grid.z = routed slots; GRP_TOKEN:
// grid.z = tokens): mb 1, stages 2, up to 16 waves; fp16 / bf16 / fp8
// activations.
int launch_skinny_byslot(int fmt, int mode, const SkinnyCfg& cfg, const SkinnyArgs& a, int64_t blocks,
                         void* stream);
int launch_moe_align(int64_t t, int topk, int num_experts, int block_m, const int32_t* ids, int32_t* sorted_ids,
                     int32_t* block_expert, int32_t* num_padded, void* stream);
// Per-row fp8 requantisation of the gate_up epilogue's fp32 rows; with null
// sorted_ids and num_padded the rows are the slots themselves (max_rows of them).
int launch_moe_requant(const float* act32, const int32_t* sorted_ids, const int32_t* num_padded, int n_slots,
                       int inter, int64_t max_rows, uint8_t* codes, float* scales, void* stream);
// y[t][col0 + c] = RNE(sum over the token's topk weighted slot rows), rows
// [t*topk][ncol] bf16 (summed in fp32 in slot order), c < ncol; y row stride n.
int launch_moe_combine(const uint16_t* rows, int topk, int64_t t, int64_t n, int64_t col0, int64_t ncol, void* y,
                       int out_bf16, void* stream);
#endif  // __HIPCC_RTC__

struct TiledArgs {
  const void* a;
  const float* a_scale;
  const uint8_t* a_e8m0;  // MXFP4 activations: E8M0 words [K/128][M][4]
  const void* w;
  const void* scales;
  const uint32_t* zeros;
  const uint8_t* e8m0;
  const float* tscale;  // NVFP4: the fp32 tensor scale (device)
  void* out;
  int M, N, K, G;
  int zp_fixed;
  int scale_bf16;
  int out_bf16;
  int tiles_m, tiles_n;
  int group_m;  // dense launch order: row tiles per group (>= 1)
  int gps;      // groups per split (dense)
  float* part;  // [split][M][N] fp32 partials, or null (no split)
  // ---- grouped (MoE) mode: the same fields as SkinnyArgs ----
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  const float* topk_w;
  int topk;
  int n_slots;
  int epi;
  int half_nblk;
  int64_t w_expert, s_expert, z_expert, e8_expert;
  float* f32_out;    // gate_up fp32 act (QFP8)
  uint16_t* rows16;  // down: weighted slot rows, bf16 [n_slots][N]
};

#ifndef __HIPCC_RTC__
int launch_tiled(int fmt, const TiledCfgRt& cfg, const TiledArgs& a, void* stream);
// Grouped launch: grid (n tiles, aligned blocks of bm rows).
int launch_tiled_grouped(int fmt, int mode, const TiledCfgRt& cfg, const TiledArgs& a, int64_t blocks,
                         void* stream);
// out[i] = round(sum_s part[s * mn + i]) in index order (fp16 / bf16 out).
int launch_splitk_reduce(const float* part, int splits, int64_t mn, void* out, int out_bf16, void* stream);
// Size of the library-owned device scratch of hq_gemm_noalloc, and its address
// on the current device (looked up once per device; a hipError_t).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
int noalloc_scratch(void** ptr);
int launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, void* stream);
int launch_mfma_peak(int dtype, int workgroups, int iters, uint32_t* sink, void* stream);
double mfma_peak_flops(int dtype, int workgroups, int iters);
// Per-row quantiser: x [m, k] fp16/bf16 -> codes [m, k] (fp8 e4m3 or int8)
// and scales [m]; k a multiple of 8.
int launch_quantize_rows(int64_t m, int64_t k, int in_bf16, int out_fp8, const void* x, void* codes, float* scales,
                         void* stream);
// MXFP4 block quantiser: x [m, k] fp16/bf16 -> codes [m, k/2] bytes and E8M0
// words [k/128][m][4]; k a multiple of 128.
int launch_quantize_mx(int64_t m, int64_t k, int in_bf16, const void* x, void* codes, uint8_t* e8m0, void* stream);

// Pending timing events for the next launch on this thread (see
// hq_time_next_launch); take_timing() returns and clears them.
struct TimingEvents {
  void* start;
  void* stop;
};
TimingEvents take_timing();
// Arms the events the next launch takes (either may be null).
void arm_timing(TimingEvents t);
int launch_repack(const hq_plan* p, const void* codes, const void* scales, const void* zx,
                  void* w_out, void* meta_out, void* stream);
#endif  // __HIPCC_RTC__

}  // namespace hq
