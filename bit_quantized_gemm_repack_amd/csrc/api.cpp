// C ABI of the quantized GEMM library: descriptors, validation, the
// execution-choice heuristic and kernel dispatch.
//
// The split between a quantisation description (what the bits mean) and an
// execution choice (tile shape, pipeline depth, matrix instruction), chosen
// by a rule-based heuristic that a caller may override, follows the Humming
// page on news.ditty.ir (summary: layer / compute / tuning configs; the
// heuristic is rule-based) and cocoloop.cn (limits section: tuning is
// heuristic, not autotuned).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <new>
#include <string>

#include "hq_internal.h"
#include "jit.h"

namespace {

thread_local std::string g_last_error;
thread_local hq::TimingEvents g_timing{nullptr, nullptr};

hq_status fail(hq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hq_status fail(hq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

hq_status ok() {
  g_last_error.clear();
  return HQ_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Map a quantisation description to a kernel format, or fail.
hq_status classify(const hq_quant_desc& q, int* fmt) {
  if (q.out != HQ_F16 && q.out != HQ_BF16)
    return fail(HQ_ERR_UNSUPPORTED, "output dtype must be fp16 or bf16");
  if (q.w_elem == HQ_U8) {
    if (q.w_bits != 8) return fail(HQ_ERR_UNSUPPORTED, "U8 weights have w_bits 8 (got %d)", q.w_bits);
    if (q.group_size != 128) return fail(HQ_ERR_UNSUPPORTED, "INT8 weights need group_size 128 (got %d)", q.group_size);
    if (q.scale != HQ_F16 && q.scale != HQ_BF16)
      return fail(HQ_ERR_UNSUPPORTED, "INT8 group scales must be fp16 or bf16");
    if (q.zp != HQ_ZP_FIXED) return fail(HQ_ERR_UNSUPPORTED, "INT8 weights are implemented with a fixed zero point");
    if (q.zp_value < 0 || q.zp_value > 255) return fail(HQ_ERR_INVALID_ARG, "INT8 fixed zero point must be 0..255");
    if ((q.act != HQ_F16 && q.act != HQ_BF16) || q.act_scale != HQ_ASCALE_NONE)
      return fail(HQ_ERR_UNSUPPORTED, "INT8 weights are implemented with fp16 / bf16 activations");
    *fmt = q.act == HQ_F16 ? hq::FMT_W8F16 : hq::FMT_W8BF16;
    return HQ_OK;
  }
  if (q.w_elem == HQ_I4) {
    if (q.w_bits != 4) return fail(HQ_ERR_UNSUPPORTED, "MXINT4 elements have w_bits 4 (got %d)", q.w_bits);
    if (q.group_size != 32 || q.scale != HQ_E8M0 || q.zp != HQ_ZP_NONE)
      return fail(HQ_ERR_UNSUPPORTED, "MXINT4 weights take one E8M0 scale per 32 k and no zero point");
    if ((q.act != HQ_F16 && q.act != HQ_BF16) || q.act_scale != HQ_ASCALE_NONE)
      return fail(HQ_ERR_UNSUPPORTED, "MXINT4 weights are implemented with fp16 / bf16 activations");
    *fmt = q.act == HQ_F16 ? hq::FMT_MX4F16 : hq::FMT_MX4BF16;
    return HQ_OK;
  }
  if (q.w_elem == HQ_U2 || q.w_elem == HQ_U3) {
    const int bits = q.w_elem == HQ_U2 ? 2 : 3;
    if (q.w_bits != bits) return fail(HQ_ERR_UNSUPPORTED, "U%d weights have w_bits %d (got %d)", bits, bits, q.w_bits);
    if (q.group_size != 128)
      return fail(HQ_ERR_UNSUPPORTED, "INT%d weights need group_size 128 (got %d)", bits, q.group_size);
    if (q.scale != HQ_F16 && q.scale != HQ_BF16)
      return fail(HQ_ERR_UNSUPPORTED, "INT%d group scales must be fp16 or bf16", bits);
    if (q.zp != HQ_ZP_FIXED)
      return fail(HQ_ERR_UNSUPPORTED, "INT%d weights are implemented with a fixed zero point", bits);
    if (q.zp_value < 0 || q.zp_value >= (1 << bits))
      return fail(HQ_ERR_INVALID_ARG, "INT%d fixed zero point must be 0..%d", bits, (1 << bits) - 1);
    if ((q.act != HQ_F16 && q.act != HQ_BF16) || q.act_scale != HQ_ASCALE_NONE)
      return fail(HQ_ERR_UNSUPPORTED, "INT%d weights are implemented with fp16 / bf16 activations", bits);
    if (bits == 2) *fmt = q.act == HQ_F16 ? hq::FMT_W2F16 : hq::FMT_W2BF16;
    else *fmt = q.act == HQ_F16 ? hq::FMT_W3F16 : hq::FMT_W3BF16;
    return HQ_OK;
  }
  if (q.w_bits != 4) return fail(HQ_ERR_UNSUPPORTED, "this weight element needs w_bits 4 (got %d)", q.w_bits);
  if (q.w_elem == HQ_U4) {
    if (q.group_size != 128) return fail(HQ_ERR_UNSUPPORTED, "INT4 weights need group_size 128 (got %d)", q.group_size);
    if (q.scale != HQ_F16 && q.scale != HQ_BF16)
      return fail(HQ_ERR_UNSUPPORTED, "INT4 group scales must be fp16 or bf16");
    if (q.zp == HQ_ZP_FIXED) {
      if (q.zp_value < 0 || q.zp_value > 15) return fail(HQ_ERR_INVALID_ARG, "fixed zero point must be 0..15");
    } else if (q.zp != HQ_ZP_PER_GROUP_U4) {
      return fail(HQ_ERR_UNSUPPORTED, "INT4 weights need a fixed or per-group zero point");
    }
    switch (q.act) {
      case HQ_F16:
      case HQ_BF16:
        if (q.act_scale != HQ_ASCALE_NONE) return fail(HQ_ERR_UNSUPPORTED, "16-bit activations take no scale");
        *fmt = q.act == HQ_F16 ? hq::FMT_W16F16 : hq::FMT_W16BF16;
        return HQ_OK;
      case HQ_INT8:
        if (q.act_scale != HQ_ASCALE_PER_TOKEN_F32)
          return fail(HQ_ERR_UNSUPPORTED, "int8 activations need per-token fp32 scales");
        if (q.zp != HQ_ZP_FIXED || q.zp_value != 8)
          return fail(HQ_ERR_UNSUPPORTED, "INT4 x INT8 needs the symmetric zero point 8");
        *fmt = hq::FMT_I8;
        return HQ_OK;
      case HQ_FP8_E4M3:
        if (q.act_scale != HQ_ASCALE_PER_TOKEN_F32)
          return fail(HQ_ERR_UNSUPPORTED, "fp8 activations need per-token fp32 scales");
        *fmt = hq::FMT_Q8;
        return HQ_OK;
      default:
        return fail(HQ_ERR_UNSUPPORTED, "unsupported activation dtype %d for INT4 weights", (int)q.act);
    }
  }
  if (q.w_elem == HQ_FP4_E2M1 && q.scale == HQ_FP8_E4M3) {
    // NVFP4: E2M1 elements, one E4M3 scale per 16 k, an fp32 tensor scale
    if (q.w_bits != 4 || q.group_size != 16 || q.zp != HQ_ZP_NONE)
      return fail(HQ_ERR_UNSUPPORTED, "NVFP4 weights take one E4M3 scale per 16 k and no zero point");
    if ((q.act != HQ_F16 && q.act != HQ_BF16) || q.act_scale != HQ_ASCALE_NONE)
      return fail(HQ_ERR_UNSUPPORTED, "NVFP4 weights are implemented with fp16 / bf16 activations");
    *fmt = q.act == HQ_F16 ? hq::FMT_NV4F16 : hq::FMT_NV4BF16;
    return HQ_OK;
  }
  if (q.w_elem == HQ_FP4_E2M1) {
    if (q.group_size != 32) return fail(HQ_ERR_UNSUPPORTED, "MXFP4 needs block size 32");
    if (q.scale != HQ_E8M0) return fail(HQ_ERR_UNSUPPORTED, "MXFP4 needs E8M0 block scales");
    if (q.zp != HQ_ZP_NONE) return fail(HQ_ERR_UNSUPPORTED, "MXFP4 has no zero point");
    if (q.act == HQ_FP4_E2M1) {
      if (q.act_scale != HQ_ASCALE_MX_E8M0)
        return fail(HQ_ERR_UNSUPPORTED, "MXFP4 activations need E8M0 block scales (HQ_ASCALE_MX_E8M0)");
      *fmt = hq::FMT_F44;
      return HQ_OK;
    }
    if (q.act != HQ_FP8_E4M3 || q.act_scale != HQ_ASCALE_PER_TOKEN_F32)
      return fail(HQ_ERR_UNSUPPORTED, "MXFP4 weights take fp8 e4m3 per-token or MXFP4 activations");
    *fmt = hq::FMT_F4;
    return HQ_OK;
  }
  return fail(HQ_ERR_UNSUPPORTED, "unsupported weight element type %d", (int)q.w_elem);
}

const char* fmt_name(int fmt) {
  switch (fmt) {
    case hq::FMT_W16F16: return "w4a16-f16";
    case hq::FMT_W16BF16: return "w4a16-bf16";
    case hq::FMT_W8F16: return "w8a16-f16";
    case hq::FMT_W8BF16: return "w8a16-bf16";
    case hq::FMT_W2F16: return "w2a16-f16";
    case hq::FMT_W2BF16: return "w2a16-bf16";
    case hq::FMT_W3F16: return "w3a16-f16";
    case hq::FMT_W3BF16: return "w3a16-bf16";
    case hq::FMT_MX4F16: return "w4a16-mxint4-f16";
    case hq::FMT_MX4BF16: return "w4a16-mxint4-bf16";
    case hq::FMT_NV4F16: return "w4a16-nvfp4-f16";
    case hq::FMT_NV4BF16: return "w4a16-nvfp4-bf16";
    case hq::FMT_I8: return "w4a8-int8";
    case hq::FMT_Q8: return "w4a8-fp8";
    case hq::FMT_F4: return "w4a8-mxfp4";
    case hq::FMT_F44: return "w4a4-mxfp4";
  }
  return "?";
}

// The matrix-instruction operand type a kernel format runs on.
hq_mfma_in implied_mfma(int fmt) {
  switch (fmt) {
    case hq::FMT_I8: return HQ_MFMA_INT8;
    case hq::FMT_Q8: return HQ_MFMA_FP8;
    case hq::FMT_F4: return HQ_MFMA_FP8_FP4;
    case hq::FMT_F44: return HQ_MFMA_FP4;
  }
  return hq::f16_act(fmt) ? HQ_MFMA_F16 : HQ_MFMA_BF16;
}

const char* mfma_name(hq_mfma_in t) {
  switch (t) {
    case HQ_MFMA_AUTO: return "auto";
    case HQ_MFMA_F16: return "f16";
    case HQ_MFMA_BF16: return "bf16";
    case HQ_MFMA_FP8: return "fp8";
    case HQ_MFMA_INT8: return "int8";
    case HQ_MFMA_FP8_FP4: return "fp8xfp4";
    case HQ_MFMA_FP4: return "fp4";
  }
  return "?";
}

bool valid_pow(int v) { return v == 1 || v == 2 || v == 4; }

}  // namespace

namespace hq {

void arm_timing(TimingEvents t) { g_timing = t; }

TimingEvents take_timing() {
  TimingEvents t = g_timing;
  g_timing = TimingEvents{nullptr, nullptr};
  return t;
}

static const hq_tuning* tuned_for(const hq_plan* p, int64_t m) {
  for (const auto& t : p->tuned)
    if (t.first == m) return &t.second;
  return &p->user;
}

Exec choose_exec(const hq_plan* p, int64_t m, const hq_tuning* up) {
  Exec e{};
  e.kernel = KER_SKINNY;
  const int64_t N = p->layer.n;
  const int64_t G = p->layer.k / kFragK;
  const hq_tuning& u = up ? *up : *tuned_for(p, m);
  const int64_t mm = m > 0 ? m : 1;
  // Large M: the MFMA-bound tiled kernel (needs whole 128/256-column tiles);
  // from 33 rows on, the activation tile in LDS is shared by the four waves
  // instead of being re-read by every 16-column workgroup.
  const bool tiled_ok = p->compute.epi != HQ_EPI_I32_ACC && N % 128 == 0;
  // 33..64 rows of 16-bit activations (INT4 weights): 16-row x 64-column skinny blocks with
  // no K split while they fill the chip at most once (N/64 * ceil(m/16) <=
  // 256 workgroups) and at most 64 groups along K; a sweep of the decode
  // shapes on MI355X put them ahead of the split tiled kernel at N = K = 4096
  // (10.0 against 15.3 us) and behind it for wider layers (N = 14336: 28
  // against 24 us) and for longer K (K = 14336: 26.3 against 22.0 us for the
  // tiled kernel with an 8-way split, whose activation tile each workgroup
  // reads once instead of once per 16-row block)
  const bool skinny_mid = (p->fmt == FMT_W16F16 || p->fmt == FMT_W16BF16) && m > 32 && m <= 64 && N % 64 == 0 && (N / 64) * cdiv(mm, 16) <= 256 &&
                          G <= 64 && p->compute.kind == HQ_GEMM_DENSE;
  const bool tiled_auto = m > 32 && !skinny_mid;
  if (tiled_ok && (u.kernel == KER_TILED || (u.kernel == 0 && tiled_auto))) {
    e.kernel = KER_TILED;
    // Tile shapes from sweeps on MI355X (N = 4096..16384, K = 2048..8192):
    //   16-bit activations (INT2 / INT4 / INT8 weights): 128-row tiles from
    //   256 rows on; fp16 128 x 256 where that still gives 192 tiles, else
    //   128 x 128, with a 3-group pipeline; bf16 128 x 128 with a 2-group
    //   pipeline;
    //   MXFP4 weights x 8/4-bit activations from 512 rows: 64 x 128 tiles
    //   (64 x 256 once that still gives 512 tiles) with a 3-group pipeline;
    //   int8 and fp8 x INT4 64 x 128 with a 2-group pipeline.
    const bool act16 = act16_fmt(p->fmt);
    e.tl.bm = (m >= 512 || (act16 && m >= 256)) ? 128 : 64;
    e.tl.nbw = 2;
    int stages = 3;
    if (act16) {
      if (f16_act(p->fmt)) e.tl.nbw = (m >= 512 && N % 256 == 0 && cdiv(mm, 128) * (N / 256) >= 192) ? 4 : 2;
      else stages = 2;
    }
    if (!act16 && m >= 512) {
      e.tl.bm = 64;
      if (mx_weights(p->fmt)) {
        // two workgroups per CU: 64 x 128 tiles up to 512 of them, else 64 x 256
        e.tl.nbw = (N % 256 == 0 && cdiv(mm, 64) * (N / 256) >= 512) ? 4 : 2;
        stages = 3;
      } else {
        stages = 2;
      }
    }
    // Launch order: groups of 8 row tiles walked column by column (a sweep of
    // 1, 2, 4, 8 at M = 1024..4096 on MI355X: 8 best for every format, 10-19 %
    // faster than row by row, the L2 of each XCD then serving a block of tiles)
    e.tl.gm = u.tile_group ? u.tile_group : 8;
    if (u.tile_m) e.tl.bm = u.tile_m;
    if (u.tile_n) e.tl.nbw = u.tile_n / 64;
    e.tiles_m = cdiv(mm, e.tl.bm);
    e.tiles_n = e.tl.nbw > 0 ? N / (64 * e.tl.nbw) : 0;
    // Too few tiles to fill the 256 CUs: split K over workgroups (each split
    // at least two groups), partial tiles summed by a second kernel.
    int64_t split = 1;
    const int64_t tiles = e.tiles_m * e.tiles_n;
    if (u.split_k) split = u.split_k;
    else if (tiles > 0 && tiles < 256) split = std::min<int64_t>(cdiv(256, tiles), std::max<int64_t>(1, G / 2));
    if (!u.split_k && act16) {
      // 16-bit activations: no split from 192 tiles on, else a power of two
      // (an even share of the groups per split)
      if (tiles >= 192) split = 1;
      while (split & (split - 1)) split &= split - 1;
    }
    split = std::max<int64_t>(1, std::min<int64_t>(split, G));
    split = cdiv(G, cdiv(G, split));  // no empty split
    e.tl.split = (int)split;
    e.tl.stages = u.stages ? u.stages : ((u.tile_m || u.tile_n) ? 3 : stages);
    e.ws_bytes = split > 1 ? align256((size_t)split * (size_t)mm * (size_t)N * 4) : 0;
    return e;
  }
  SkinnyCfg c{};
  c.mb = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  c.nb = 1;
  if (skinny_mid && u.kernel == 0) {
    c.mb = 1;
    c.nb = 4;
  }
  // Rules from a sweep of the decode shapes on MI355X (kernel durations):
  //   wide layers (>= 512 column blocks): 4 column blocks per workgroup;
  //   otherwise one column block per workgroup with K split over the waves;
  //   8 waves, except 4 for 5..16 rows of 16-bit activations (each wave's
  //   activation loads grow with the rows and the element size); two groups
  //   of loads in flight per wave.
  c.stages = 2;
  if (c.mb == 1) {
    const bool act16 = act16_fmt(p->fmt);
    c.waves = (m <= 4 || !act16) ? 8 : 4;
    if (N / 16 >= 512 && N % 64 == 0) c.nb = 4;
    // one row of 16-bit INT4 activations (staged in LDS, so a wave's loads
    // are its weights and metadata only): 16 waves per column block over
    // long K, and two column blocks of 4 waves on wide layers (three
    // alternating runs on one MI355X host: N = 4096, K = 14336 9.44-9.63 ->
    // 9.11-9.24 us; N = 14336, K = 4096 9.10-9.19 -> 8.78-8.94 us)
    if (m == 1 && (p->fmt == FMT_W16F16 || p->fmt == FMT_W16BF16)) {
      if (c.nb == 1 && G >= 64) c.waves = 16;
      if (c.nb == 4 && N % 32 == 0) {
        c.nb = 2;
        c.waves = 4;
      }
    }
  } else {
    c.waves = 8;
  }
  c.waves = (int)std::min<int64_t>(c.waves, std::max<int64_t>(1, G));
  // 5..16 rows and long K: the activation block is re-read by every
  // column-block workgroup; 4 column blocks per workgroup cut that 4x, and
  // a 4-way K split keeps 4x the workgroups (partials summed by the reduce).
  int64_t auto_split = 1;
  if (w8_weights(p->fmt) || w2_weights(p->fmt) || w3_weights(p->fmt)) {
    // INT8 / INT2 weights (a sweep at N = 4096..16384): two column blocks per
    // workgroup from 384 column blocks on, four from 1024 on (INT8: for 5..16
    // rows only), no K split
    if (c.mb == 1) {
      c.nb = (N / 16 >= 384 && N % 32 == 0) ? 2 : 1;
      if (N / 16 >= 1024 && N % 64 == 0 && (!w8_weights(p->fmt) || m > 4)) c.nb = 4;
    }
  } else if (c.mb == 1 && m > 4 && m <= 32 && G >= 64 && N % 64 == 0 && N / 64 >= 32) {
    c.nb = 4;
    auto_split = 4;
  }
  if (u.tile_m) c.mb = u.tile_m / 16;
  if (u.tile_n) c.nb = u.tile_n / 16;
  if (u.waves) c.waves = u.waves;
  if (u.stages) c.stages = u.stages;
  // 16-wave workgroups exist for one 16 x 16 block per wave only
  if (!u.waves && c.waves > 8 && !(c.mb == 1 && c.nb == 1 && c.stages <= 4)) c.waves = 8;
  const int64_t ntiles = N / (16 * c.nb);
  const int64_t mch = cdiv(mm, 16 * c.mb);
  int64_t split = (u.tile_m || u.tile_n || u.waves) ? 1 : auto_split;
  if (u.split_k) split = u.split_k;
  if (p->compute.epi == HQ_EPI_I32_ACC) split = u.split_k ? u.split_k : 1;
  split = std::max<int64_t>(1, std::min<int64_t>(split, G));
  split = cdiv(G, cdiv(G, split));  // no empty split
  c.split = (int)split;
  e.sk = c;
  e.tiles_m = mch;
  e.tiles_n = ntiles;
  e.ws_bytes = 0;
  if (c.split > 1 && p->compute.epi != HQ_EPI_I32_ACC)
    e.ws_bytes = align256((size_t)c.split * (size_t)mm * (size_t)N * 4);
  return e;
}

}  // namespace hq

namespace {

hq_status check_exec(const hq_plan* p, const hq::Exec& e) {
  if (p->user.split_k < 0 || p->user.split_k > 64) return fail(HQ_ERR_INVALID_ARG, "split_k must be 1..64");
  if (e.kernel == hq::KER_TILED) {
    if (e.tl.bm != 64 && e.tl.bm != 128) return fail(HQ_ERR_INVALID_ARG, "tiled kernel: tile_m must be 64 or 128");
    if (e.tl.nbw != 2 && e.tl.nbw != 4) return fail(HQ_ERR_INVALID_ARG, "tiled kernel: tile_n must be 128 or 256");
    if (p->layer.n % (64 * e.tl.nbw)) return fail(HQ_ERR_INVALID_ARG, "tiled kernel: N must be a multiple of tile_n");
    if (e.tiles_m * e.tiles_n > (int64_t(1) << 31) - 1) return fail(HQ_ERR_UNSUPPORTED, "too many tiles");
    if (e.tl.split < 1 || e.tl.split > 64) return fail(HQ_ERR_INVALID_ARG, "split_k must be 1..64");
    if (e.tl.gm < 1 || e.tl.gm > 64) return fail(HQ_ERR_INVALID_ARG, "tiled kernel: tile_group must be 1..64");
    {
      // load pipeline: stages x (tile_m rows x one group of A) in LDS, and the
      // loads of stages - 2 groups in flight within the 6-bit wait counter
      const bool act16 = hq::act16_fmt(p->fmt);
      const bool act4 = p->fmt == hq::FMT_F44;
      const int rowb = act16 ? 256 : (act4 ? 64 : 128);
      const int lps = e.tl.bm * rowb / 1024 / 4 + e.tl.nbw * (hq::e8m0_meta(p->fmt) ? 2 : 3) +
                      (act4 ? e.tl.bm / 16 : 0) + ((hq::w8_weights(p->fmt) || hq::w3_weights(p->fmt)) ? e.tl.nbw : 0);
      if (e.tl.stages < 2 || e.tl.stages > 5) return fail(HQ_ERR_INVALID_ARG, "tiled kernel: stages must be 2..5");
      if (e.tl.stages * e.tl.bm * rowb > 160 * 1024 || lps * (e.tl.stages - 2) >= 64)
        return fail(HQ_ERR_INVALID_ARG, "tiled kernel: too many stages for this tile");
    }
    return HQ_OK;
  }
  const hq::SkinnyCfg& c = e.sk;
  if (!valid_pow(c.mb)) return fail(HQ_ERR_INVALID_ARG, "tile_m must be 16, 32 or 64");
  if (!valid_pow(c.nb)) return fail(HQ_ERR_INVALID_ARG, "tile_n must be 16, 32 or 64");
  if (p->layer.n % (16 * c.nb)) return fail(HQ_ERR_INVALID_ARG, "N must be a multiple of tile_n");
  if (c.waves < 1 || c.waves > 16) return fail(HQ_ERR_INVALID_ARG, "waves must be 1..16");
  if (c.waves > 8 && (c.mb != 1 || c.nb != 1 || c.stages > 4))
    return fail(HQ_ERR_INVALID_ARG, "more than 8 waves needs tile_m=16, tile_n=16 and stages <= 4");
  if (c.stages != 2 && c.stages != 4 && c.stages != 8) return fail(HQ_ERR_INVALID_ARG, "stages must be 2, 4 or 8");
  if (c.stages == 8 && (c.mb != 1 || c.nb > 2)) return fail(HQ_ERR_INVALID_ARG, "stages=8 needs tile_m=16, tile_n<=32");
  if (c.split < 1 || c.split > 64) return fail(HQ_ERR_INVALID_ARG, "split_k must be 1..64");
  if ((size_t)c.waves * c.mb * c.nb * 4 * 64 * 4 > 32768)
    return fail(HQ_ERR_INVALID_ARG, "waves * tile_m * tile_n too large for the reduction buffer");
  // register budget: these shapes would spill at two waves per SIMD
  const bool act16 = hq::act16_fmt(p->fmt);
  if ((c.stages < 8 && c.mb * c.nb * c.stages > 16) || c.mb * c.stages > 8 || (c.mb == 4 && c.nb == 2 && act16) ||
      (hq::w8_weights(p->fmt) && c.mb * c.nb * c.stages > 8))
    return fail(HQ_ERR_INVALID_ARG, "tile_m/tile_n/stages combination exceeds the register budget");
  return HQ_OK;
}

}  // namespace

extern "C" {

int hq_abi_version(void) { return HQ_ABI_VERSION; }

const char* hq_status_str(hq_status s) {
  switch (s) {
    case HQ_OK: return "HQ_OK";
    case HQ_ERR_INVALID_ARG: return "HQ_ERR_INVALID_ARG";
    case HQ_ERR_UNSUPPORTED: return "HQ_ERR_UNSUPPORTED";
    case HQ_ERR_WORKSPACE: return "HQ_ERR_WORKSPACE";
    case HQ_ERR_HIP: return "HQ_ERR_HIP";
    case HQ_ERR_INTERNAL: return "HQ_ERR_INTERNAL";
  }
  return "HQ_ERR_UNKNOWN";
}

const char* hq_last_error(void) { return g_last_error.c_str(); }

hq_status hq_time_next_launch(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(HQ_ERR_INVALID_ARG, "give both events or neither");
  g_timing = hq::TimingEvents{start_event, stop_event};
  return ok();
}

hq_status hq_plan_create(const hq_layer_desc* layer, const hq_compute* compute, int64_t max_m,
                         const hq_tuning* tuning, hq_plan** out) {
  try {
    if (!layer || !compute || !out) return fail(HQ_ERR_INVALID_ARG, "null argument");
    *out = nullptr;
    if (layer->n <= 0 || layer->k <= 0) return fail(HQ_ERR_INVALID_ARG, "n and k must be positive");
    if (layer->n % 16) return fail(HQ_ERR_UNSUPPORTED, "N must be a multiple of 16 (got %lld)", (long long)layer->n);
    if (layer->k % 128) return fail(HQ_ERR_UNSUPPORTED, "K must be a multiple of 128 (got %lld)", (long long)layer->k);
    if (layer->n > (1 << 24) || layer->k > (1 << 24)) return fail(HQ_ERR_UNSUPPORTED, "N or K too large");
    if (max_m < 0 || max_m > (1 << 20)) return fail(HQ_ERR_INVALID_ARG, "max_m out of range");
    if (layer->num_experts < 1) return fail(HQ_ERR_INVALID_ARG, "num_experts must be >= 1");
    if (compute->kind != HQ_GEMM_DENSE && compute->kind != HQ_GEMM_GROUPED)
      return fail(HQ_ERR_INVALID_ARG, "unknown GEMM kind");
    if (compute->kind == HQ_GEMM_DENSE && layer->num_experts != 1)
      return fail(HQ_ERR_INVALID_ARG, "a dense plan has exactly one expert");
    int fmt = 0;
    hq_status s = classify(layer->q, &fmt);
    if (s != HQ_OK) return s;
    if (compute->mfma_in < HQ_MFMA_AUTO || compute->mfma_in > HQ_MFMA_FP4)
      return fail(HQ_ERR_INVALID_ARG, "unknown matrix-instruction type %d", (int)compute->mfma_in);
    if (compute->mfma_in != HQ_MFMA_AUTO && compute->mfma_in != implied_mfma(fmt))
      return fail(HQ_ERR_UNSUPPORTED, "%s runs on the %s matrix instruction, not %s", fmt_name(fmt),
                  mfma_name(implied_mfma(fmt)), mfma_name(compute->mfma_in));
    switch (compute->epi) {
      case HQ_EPI_NONE: break;
      case HQ_EPI_I32_ACC:
        if (fmt != hq::FMT_I8 || compute->kind != HQ_GEMM_DENSE)
          return fail(HQ_ERR_UNSUPPORTED, "int32 accumulator output needs a dense INT4 x INT8 plan");
        break;
      case HQ_EPI_SILU_MUL:
      case HQ_EPI_SILU_MUL_QFP8:
      case HQ_EPI_TOPK_COMBINE:
        if (compute->kind != HQ_GEMM_GROUPED)
          return fail(HQ_ERR_UNSUPPORTED, "grouped epilogues are not available on dense plans");
        break;
      default:
        return fail(HQ_ERR_INVALID_ARG, "unknown epilogue");
    }
    if (compute->kind == HQ_GEMM_GROUPED) {
      if (fmt != hq::FMT_W16F16 && fmt != hq::FMT_W16BF16 && fmt != hq::FMT_Q8)
        return fail(HQ_ERR_UNSUPPORTED, "grouped GEMM supports INT4 weights with fp16/bf16/fp8 activations");
      if ((compute->epi == HQ_EPI_SILU_MUL || compute->epi == HQ_EPI_SILU_MUL_QFP8) && layer->n % 32)
        return fail(HQ_ERR_UNSUPPORTED, "SiLU * mul needs n (gate + up) a multiple of 32");
      if (compute->epi == HQ_EPI_TOPK_COMBINE && layer->n % 64)
        return fail(HQ_ERR_UNSUPPORTED, "the combining down GEMM needs n a multiple of 64");
      if (tuning) {
        const int tm = tuning->tile_m, tn = tuning->tile_n;
        if (tm != 0 && tm != 16 && tm != 32 && tm != 64 && tm != 128)
          return fail(HQ_ERR_UNSUPPORTED, "grouped tile_m must be 16 or 32 (skinny), 64 or 128 (tiled)");
        if (tuning->kernel == hq::KER_SKINNY && tm > 32)
          return fail(HQ_ERR_UNSUPPORTED, "the skinny grouped kernel uses 16- or 32-row blocks");
        if (tuning->kernel == hq::KER_TILED && (tm == 16 || tm == 32))
          return fail(HQ_ERR_UNSUPPORTED, "the tiled grouped kernel uses 64- or 128-row blocks");
        if (tn != 0 && tn != 16 && tn != 32 && tn != 64 && tn != 128 && tn != 256)
          return fail(HQ_ERR_UNSUPPORTED, "grouped tile_n must be 128 or 256 (tiled), 16, 32 or 64 (by slot)");
        if (tuning->waves < 0 || tuning->waves > 16) return fail(HQ_ERR_UNSUPPORTED, "grouped waves must be 1..16");
        if (tn != 0 && layer->n % tn) return fail(HQ_ERR_UNSUPPORTED, "n must be a multiple of tile_n");
      }
    }
    hq_plan* p = new (std::nothrow) hq_plan();
    if (!p) return fail(HQ_ERR_INTERNAL, "out of host memory");
    p->layer = *layer;
    p->compute = *compute;
    p->max_m = max_m;
    if (tuning) p->user = *tuning;
    p->fmt = fmt;
    const int64_t N = layer->n, K = layer->k, G = K / 128;
    p->w_bytes_per_expert = (size_t)N * (size_t)K * (size_t)hq::frag_bytes(fmt) / (size_t)(hq::kFragN * hq::kFragK);
    if (hq::nvfp4_weights(fmt)) {
      p->scale_region_bytes = 0;  // E4M3 region, then the fp32 tensor scale (16 bytes)
      p->meta_bytes_per_expert = (size_t)(N * K / 16 + 16);
    } else if (hq::e8m0_meta(fmt)) {
      p->scale_region_bytes = 0;
      p->meta_bytes_per_expert = (size_t)(N * K / 32);
    } else {
      p->scale_region_bytes = (size_t)(N * G * 2);
      p->meta_bytes_per_expert = p->scale_region_bytes;
      if (layer->q.zp == HQ_ZP_PER_GROUP_U4) p->meta_bytes_per_expert += (size_t)((N / 16) * G * 8);
    }
    hq::Exec e = hq::choose_exec(p, max_m > 0 ? max_m : 1);
    s = compute->kind == HQ_GEMM_GROUPED ? HQ_OK : check_exec(p, e);
    if (s != HQ_OK) {
      delete p;
      return s;
    }
    *out = p;
    return ok();
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_plan_create");
  }
}

hq_status hq_plan_destroy(hq_plan* plan) {
  delete plan;
  return ok();
}

static hq_status describe_grouped(const hq_plan* p, int64_t slots, char* buf, size_t len);

hq_status hq_plan_describe(const hq_plan* p, int64_t m, char* buf, size_t len) {
  if (!p || !buf || len == 0) return fail(HQ_ERR_INVALID_ARG, "null argument");
  if (m < 1) m = 1;
  if (p->compute.kind == HQ_GEMM_GROUPED) return describe_grouped(p, m, buf, len);
  hq::Exec e = hq::choose_exec(p, m);
  if (e.kernel == hq::KER_TILED) {
    snprintf(buf, len,
             "kernel=tiled fmt=%s mfma=%s m=%lld n=%lld k=%lld tile_m=%d tile_n=%d waves=4 split_k=%d stages=%d "
             "tile_group=%d grid=%lldx%d ws=%zu",
             fmt_name(p->fmt), mfma_name(implied_mfma(p->fmt)), (long long)m, (long long)p->layer.n,
             (long long)p->layer.k, e.tl.bm, 64 * e.tl.nbw, e.tl.split, e.tl.stages, e.tl.gm,
             (long long)(e.tiles_m * e.tiles_n), e.tl.split, e.ws_bytes);
    return ok();
  }
  snprintf(buf, len,
           "kernel=skinny fmt=%s mfma=%s m=%lld n=%lld k=%lld tile_m=%d tile_n=%d waves=%d split_k=%d stages=%d "
           "grid=%lldx%dx%lld ws=%zu",
           fmt_name(p->fmt), mfma_name(implied_mfma(p->fmt)), (long long)m, (long long)p->layer.n,
           (long long)p->layer.k, 16 * e.sk.mb, 16 * e.sk.nb, e.sk.waves, e.sk.split, e.sk.stages,
           (long long)e.tiles_n, e.sk.split, (long long)e.tiles_m, e.ws_bytes);
  return ok();
}

hq_status hq_plan_workspace_bytes(const hq_plan* p, int64_t m, size_t* bytes) {
  if (!p || !bytes) return fail(HQ_ERR_INVALID_ARG, "null argument");
  if (m < 0 || m > p->max_m) return fail(HQ_ERR_INVALID_ARG, "m out of range [0, max_m]");
  *bytes = m == 0 ? 0 : hq::choose_exec(p, m).ws_bytes;
  return ok();
}

hq_status hq_repacked_bytes(const hq_plan* p, size_t* w_bytes, size_t* meta_bytes) {
  if (!p || !w_bytes || !meta_bytes) return fail(HQ_ERR_INVALID_ARG, "null argument");
  *w_bytes = p->w_bytes_per_expert * (size_t)p->layer.num_experts;
  *meta_bytes = p->meta_bytes_per_expert * (size_t)p->layer.num_experts;
  return ok();
}

static hq_status check_repack_args(const hq_plan* p, const void* codes, const void* scales, const void* zx,
                                   const void* w_out, const void* meta_out) {
  if (!p || !codes || !w_out || !meta_out) return fail(HQ_ERR_INVALID_ARG, "null argument");
  if (hq::nvfp4_weights(p->fmt)) {
    if (!zx || !scales) return fail(HQ_ERR_INVALID_ARG, "NVFP4 repack needs the E4M3 block scales and the tensor scale");
  } else if (hq::e8m0_meta(p->fmt)) {
    if (!zx) return fail(HQ_ERR_INVALID_ARG, "MXFP4 / MXINT4 repack needs the E8M0 scales");
  } else {
    if (!scales) return fail(HQ_ERR_INVALID_ARG, "INT4 repack needs the group scales");
    if (p->layer.q.zp == HQ_ZP_PER_GROUP_U4 && !zx)
      return fail(HQ_ERR_INVALID_ARG, "per-group zero points missing");
  }
  return HQ_OK;
}

hq_status hq_repack(const hq_plan* p, const void* codes, const void* scales, const void* zx, void* w_out,
                    void* meta_out, void* stream) {
  try {
    hq_status s = check_repack_args(p, codes, scales, zx, w_out, meta_out);
    if (s != HQ_OK) return s;
    if (!aligned16(codes) || !aligned16(w_out) || !aligned16(meta_out))
      return fail(HQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    int err = hq::launch_repack(p, codes, scales, zx, w_out, meta_out, stream);
    if (err != hipSuccess) return fail(HQ_ERR_HIP, "repack launch: %s", hipGetErrorString((hipError_t)err));
    return ok();
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_repack");
  }
}

hq_status hq_repack_host(const hq_plan* p, const void* codes, const void* scales, const void* zx, void* w_out,
                         void* meta_out) {
  try {
    hq_status s = check_repack_args(p, codes, scales, zx, w_out, meta_out);
    if (s != HQ_OK) return s;
    const int64_t N = p->layer.n, K = p->layer.k, E = p->layer.num_experts, G = K / 128;
    uint32_t* wo = static_cast<uint32_t*>(w_out);
    if (hq::w3_weights(p->fmt)) {
      const int64_t wpe3 = N * K * 3 / 32;
      const uint32_t* cw = static_cast<const uint32_t*>(codes);
      for (int64_t e = 0; e < E; ++e)
        for (int64_t i = 0; i < wpe3; ++i) wo[e * wpe3 + i] = hq::repack_word3(cw + e * wpe3, K, i);
    } else if (hq::w2_weights(p->fmt)) {
      const int64_t wpe2 = N * K / 16;
      const uint32_t* cw = static_cast<const uint32_t*>(codes);
      for (int64_t e = 0; e < E; ++e)
        for (int64_t i = 0; i < wpe2; ++i) wo[e * wpe2 + i] = hq::repack_word2(cw + e * wpe2, K, i);
    } else if (hq::w8_weights(p->fmt)) {
      const int64_t wpe8 = N * K / 4;
      const uint8_t* cb = static_cast<const uint8_t*>(codes);
      for (int64_t e = 0; e < E; ++e)
        for (int64_t i = 0; i < wpe8; ++i) wo[e * wpe8 + i] = hq::repack_word8(cb + e * N * K, K, i);
    } else {
      const int64_t wpe = N * K / 8;
      const uint32_t* cw = static_cast<const uint32_t*>(codes);
      for (int64_t e = 0; e < E; ++e)
        for (int64_t i = 0; i < wpe; ++i) wo[e * wpe + i] = hq::repack_word(cw + e * wpe, K, p->fmt, i);
    }
    uint8_t* meta = static_cast<uint8_t*>(meta_out);
    if (hq::nvfp4_weights(p->fmt)) {
      const int64_t per = N * K / 16;
      const uint8_t* src = static_cast<const uint8_t*>(zx);
      for (int64_t e = 0; e < E; ++e) {
        uint8_t* me = meta + e * (int64_t)p->meta_bytes_per_expert;
        for (int64_t i = 0; i < per; ++i) me[i] = src[e * per + hq::e4m3_src_index(K, i)];
        std::memset(me + per, 0, 16);
        std::memcpy(me + per, static_cast<const float*>(scales) + e, 4);
      }
      return ok();
    }
    if (hq::e8m0_meta(p->fmt)) {
      const int64_t per = N * K / 32;
      const uint8_t* src = static_cast<const uint8_t*>(zx);
      const bool cols = hq::mxint4_weights(p->fmt);
      for (int64_t e = 0; e < E; ++e)
        for (int64_t i = 0; i < per; ++i)
          meta[e * per + i] = src[e * per + (cols ? hq::e8m0_cols_src_index(K, i) : hq::e8m0_src_index(K, i))];
      return ok();
    }
    const int64_t sper = N * G;
    const uint16_t* ss = static_cast<const uint16_t*>(scales);
    uint16_t* so = reinterpret_cast<uint16_t*>(meta);
    for (int64_t e = 0; e < E; ++e)
      for (int64_t i = 0; i < sper; ++i) so[e * sper + i] = ss[e * sper + hq::scale_src_index(G, i)];
    if (p->layer.q.zp == HQ_ZP_PER_GROUP_U4) {
      const int64_t zwpe = (N / 16) * G * 2;
      const uint8_t* zs = static_cast<const uint8_t*>(zx);
      uint32_t* zo = reinterpret_cast<uint32_t*>(meta + p->scale_region_bytes * E);
      for (int64_t e = 0; e < E; ++e)
        for (int64_t i = 0; i < zwpe; ++i) zo[e * zwpe + i] = hq::zeros_word(zs + e * N * G, G, i);
    }
    return ok();
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_repack_host");
  }
}

namespace {

// Argument checks of a dense call (hq_gemm, hq_plan_autotune); m >= 1.
hq_status dense_args_check(const hq_plan* p, int64_t m, const void* a, const void* a_scale, const void* w,
                           const void* meta, void* out) {
  if (!p) return fail(HQ_ERR_INVALID_ARG, "null plan");
  if (p->compute.kind != HQ_GEMM_DENSE) return fail(HQ_ERR_INVALID_ARG, "hq_gemm needs a dense plan");
  if (m < 0 || m > p->max_m) return fail(HQ_ERR_INVALID_ARG, "m=%lld out of range [0, %lld]", (long long)m,
                                         (long long)p->max_m);
  if (!a || !w || !meta || !out) return fail(HQ_ERR_INVALID_ARG, "null device pointer");
  if (!aligned16(a) || !aligned16(w) || !aligned16(meta) || !aligned16(out))
    return fail(HQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  const bool act4 = p->fmt == hq::FMT_F44;
  const bool act8 = p->fmt == hq::FMT_I8 || p->fmt == hq::FMT_Q8 || p->fmt == hq::FMT_F4;
  if (act8 && !a_scale) return fail(HQ_ERR_INVALID_ARG, "8-bit activations need a_scale");
  if (act4 && !a_scale) return fail(HQ_ERR_INVALID_ARG, "MXFP4 activations need their E8M0 scales in a_scale");
  if (act4 && !aligned16(a_scale)) return fail(HQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  if (!act8 && !act4 && a_scale) return fail(HQ_ERR_INVALID_ARG, "16-bit activations take no a_scale");
  return HQ_OK;
}

// One dense GEMM with the execution choice e (arguments already checked).
hq_status dense_run(const hq_plan* p, const hq::Exec& e, int64_t m, const void* a, const void* a_scale,
                    const void* w, const void* meta, void* out, void* ws, size_t ws_bytes, void* stream,
                    const hq::TimingEvents& ev) {
  {
    const bool act4 = p->fmt == hq::FMT_F44;
    const bool act8 = p->fmt == hq::FMT_I8 || p->fmt == hq::FMT_Q8 || p->fmt == hq::FMT_F4;
    const float* a_scale_f = act8 ? static_cast<const float*>(a_scale) : nullptr;
    const uint8_t* a_e8m0 = act4 ? static_cast<const uint8_t*>(a_scale) : nullptr;
    hq_status s = check_exec(p, e);
    if (s != HQ_OK) return s;
    if (e.ws_bytes > 0) {
      if (!ws) return fail(HQ_ERR_WORKSPACE, "this call needs %zu workspace bytes", e.ws_bytes);
      if (ws_bytes < e.ws_bytes)
        return fail(HQ_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, e.ws_bytes);
      if (!aligned16(ws)) return fail(HQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    const int64_t N = p->layer.n, K = p->layer.k, G = K / 128;
    if (m * K > (int64_t(1) << 40)) return fail(HQ_ERR_UNSUPPORTED, "problem too large");
    const uint32_t* zeros = p->layer.q.zp == HQ_ZP_PER_GROUP_U4
                                ? reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(meta) +
                                                                    p->scale_region_bytes)
                                : nullptr;
    {
      // the kernels address A and W through 32-bit buffer ranges
      const int64_t act_bytes2 = hq::act16_fmt(p->fmt) ? 4 : (act4 ? 1 : 2);
      if (m * K * act_bytes2 / 2 >= (int64_t(1) << 31) || (int64_t)p->w_bytes_per_expert >= (int64_t(1) << 31))
        return fail(HQ_ERR_UNSUPPORTED, "activations and weights must each stay below 2 GiB");
    }
    if (e.kernel == hq::KER_TILED) {
      hq::TiledArgs t{};
      t.a = a;
      t.a_scale = a_scale_f;
      t.a_e8m0 = a_e8m0;
      t.w = w;
      if (hq::e8m0_meta(p->fmt)) t.e8m0 = static_cast<const uint8_t*>(meta);
      if (hq::nvfp4_weights(p->fmt))
        t.tscale = reinterpret_cast<const float*>(static_cast<const uint8_t*>(meta) + N * K / 16);
      else t.scales = meta;
      t.zeros = zeros;
      t.out = out;
      t.M = (int)m;
      t.N = (int)N;
      t.K = (int)K;
      t.G = (int)G;
      t.zp_fixed = p->layer.q.zp == HQ_ZP_FIXED ? p->layer.q.zp_value : -1;
      t.scale_bf16 = p->layer.q.scale == HQ_BF16;
      t.out_bf16 = p->layer.q.out == HQ_BF16;
      t.tiles_m = (int)e.tiles_m;
      t.tiles_n = (int)e.tiles_n;
      t.group_m = (int)std::min<int64_t>(e.tl.gm, std::max<int64_t>(1, e.tiles_m));
      t.gps = (int)cdiv(G, e.tl.split);
      t.part = e.tl.split > 1 ? static_cast<float*>(ws) : nullptr;
      hq::arm_timing({ev.start, e.tl.split > 1 ? nullptr : ev.stop});
      std::string jit_err;
      int err = p->jit ? hq::jit::launch_tiled(p, e.tl, t, stream, &jit_err) : hq::launch_tiled(p->fmt, e.tl, t, stream);
      if (!jit_err.empty()) {
        hq::arm_timing({nullptr, nullptr});
        return fail(HQ_ERR_UNSUPPORTED, "%s", jit_err.c_str());
      }
      if (err == hipSuccess && e.tl.split > 1) {
        hq::arm_timing({nullptr, ev.stop});
        err = hq::launch_splitk_reduce(t.part, e.tl.split, m * N, out, t.out_bf16, stream);
      }
      hq::arm_timing({nullptr, nullptr});
      if (err != hipSuccess) return fail(HQ_ERR_HIP, "gemm launch: %s", hipGetErrorString((hipError_t)err));
      return ok();
    }
    hq::SkinnyArgs args{};
    args.a = a;
    args.a_scale = a_scale_f;
    args.a_e8m0 = a_e8m0;
    args.w = w;
    if (hq::e8m0_meta(p->fmt)) {
      args.e8m0 = static_cast<const uint8_t*>(meta);
      if (hq::nvfp4_weights(p->fmt))
        args.tscale = reinterpret_cast<const float*>(static_cast<const uint8_t*>(meta) + N * K / 16);
    } else {
      args.scales = meta;
      args.zeros = zeros;
    }
    args.out = out;
    if (e.ws_bytes > 0) args.part = static_cast<float*>(ws);
    args.M = (int)m;
    args.N = (int)N;
    args.K = (int)K;
    args.G = (int)G;
    args.zp_fixed = p->layer.q.zp == HQ_ZP_FIXED ? p->layer.q.zp_value : -1;
    args.scale_bf16 = p->layer.q.scale == HQ_BF16;
    args.out_bf16 = p->layer.q.out == HQ_BF16;
    args.i32_out = p->compute.epi == HQ_EPI_I32_ACC;
    args.gps = (int)cdiv(G, e.sk.split);
    const bool reduce = e.ws_bytes > 0;
    hq::arm_timing({ev.start, reduce ? nullptr : ev.stop});
    std::string jit_err;
    int err = p->jit ? hq::jit::launch_skinny(p, e.sk, args, stream, &jit_err) : hq::launch_skinny(p->fmt, e.sk, args, stream);
    if (!jit_err.empty()) {
      hq::arm_timing({nullptr, nullptr});
      return fail(HQ_ERR_UNSUPPORTED, "%s", jit_err.c_str());
    }
    if (err == hipSuccess && reduce) {
      hq::arm_timing({nullptr, ev.stop});
      err = hq::launch_splitk_reduce(args.part, e.sk.split, m * N, out, args.out_bf16, stream);
    }
    hq::arm_timing({nullptr, nullptr});
    if (err != hipSuccess) return fail(HQ_ERR_HIP, "gemm launch: %s", hipGetErrorString((hipError_t)err));
    return ok();
  }
}

}  // namespace

hq_status hq_gemm(const hq_plan* p, int64_t m, const void* a, const void* a_scale, const void* w,
                  const void* meta, void* out, void* ws, size_t ws_bytes, void* stream) {
  const hq::TimingEvents ev = hq::take_timing();  // consumed by this call whatever happens
  try {
    if (!p) return fail(HQ_ERR_INVALID_ARG, "null plan");
    if (m == 0 && p->compute.kind == HQ_GEMM_DENSE) return ok();
    hq_status s = dense_args_check(p, m, a, a_scale, w, meta, out);
    if (s != HQ_OK) return s;
    return dense_run(p, hq::choose_exec(p, m), m, a, a_scale, w, meta, out, ws, ws_bytes, stream, ev);
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_gemm");
  }
}

hq_status hq_gemm_noalloc(const hq_plan* p, int64_t m, const void* a, const void* a_scale, const void* w,
                          const void* meta, void* out, void* stream) {
  const hq::TimingEvents ev = hq::take_timing();  // consumed by this call whatever happens
  try {
    if (!p) return fail(HQ_ERR_INVALID_ARG, "null plan");
    if (m == 0 && p->compute.kind == HQ_GEMM_DENSE) return ok();
    hq_status s = dense_args_check(p, m, a, a_scale, w, meta, out);
    if (s != HQ_OK) return s;
    const hq::Exec e = hq::choose_exec(p, m);
    if (e.ws_bytes > hq::kNoAllocScratchBytes)
      return fail(HQ_ERR_WORKSPACE,
                  "this call's split-K partials need %zu bytes, above the %zu-byte library scratch of "
                  "hq_gemm_noalloc (use hq_gemm with a workspace, or a tuning with a smaller K split)",
                  e.ws_bytes, hq::kNoAllocScratchBytes);
    void* scratch = nullptr;
    if (e.ws_bytes > 0) {
      const int err = hq::noalloc_scratch(&scratch);
      if (err != hipSuccess)
        return fail(HQ_ERR_HIP, "library scratch lookup: %s", hipGetErrorString((hipError_t)err));
    }
    return dense_run(p, e, m, a, a_scale, w, meta, out, scratch, e.ws_bytes > 0 ? hq::kNoAllocScratchBytes : 0,
                     stream, ev);
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_gemm_noalloc");
  }
}

// ---------------------------------------------------------------------------
// grouped (MoE)
// ---------------------------------------------------------------------------

// Longest possible aligned slot array: every expert's segment, plus the one
// for out-of-range ids, padded up to whole blocks.
static int64_t moe_max_padded(int64_t t, int topk, int E, int bm) {
  const int64_t raw = t * topk + (int64_t)(E + 1) * (bm - 1);
  return (raw + bm - 1) / bm * bm;
}

// Kernel choice for one grouped call.  Few slots per expert (decode-sized T)
// leave the weight stream as the cost: the skinny kernel with 16-row blocks
// reads every active expert's weights about once.  Many slots per expert make
// the GEMM MFMA-bound: the tiled kernel with 64- or 128-row blocks reuses each
// dequantised weight fragment over the whole block.
struct MoeChoice {
  bool tiled;
  int bm;  // alignment block = rows per workgroup
  hq::SkinnyCfg sk;
  hq::TiledCfgRt tl;
};

static MoeChoice moe_choice(const hq_plan* p, int64_t t, int topk) {
  MoeChoice c{};
  const hq_tuning& u = p->user;
  const int64_t N = p->layer.n;
  const double per_expert = (double)t * topk / p->layer.num_experts;
  bool tiled;
  if (u.kernel == hq::KER_TILED) tiled = true;
  else if (u.kernel == hq::KER_SKINNY) tiled = false;
  else if (u.tile_m) tiled = u.tile_m >= 64;
  else tiled = per_expert >= 12.0;  // measured crossover on MI355X (H = 7168, I = 256)
  if (tiled && N % 128) tiled = false;  // the tiled grid needs whole 128-column tiles
  c.tiled = tiled;
  if (!tiled) {
    // 16-row blocks (32 by tuning: fewer weight re-reads at ~16 slots per
    // expert, but measured slower on MI355X at T = 512)
    c.bm = (u.tile_m == 16 || u.tile_m == 32) ? u.tile_m : 16;
    c.sk.mb = c.bm / 16;
    c.sk.nb = (p->compute.epi == HQ_EPI_TOPK_COMBINE || p->compute.epi == HQ_EPI_NONE) ? 4 : 2;
    if (p->compute.epi == HQ_EPI_NONE && N % 64) c.sk.nb = 1;
    const int64_t G = p->layer.k / 128;
    c.sk.waves = (int)std::min<int64_t>(8, std::max<int64_t>(1, G));
    c.sk.stages = 2;
    c.sk.split = 1;
    return c;
  }
  c.bm = u.tile_m >= 64 ? u.tile_m : (per_expert >= 192.0 ? 128 : 64);
  int nbw;
  if (u.tile_n >= 128) nbw = u.tile_n / 64;  // smaller tile_n values are the by-slot kernel's
  else nbw = (N % 256 == 0) ? 4 : 2;
  if (N % (64 * nbw)) nbw = 2;
  c.tl.bm = c.bm;
  c.tl.nbw = nbw;
  c.tl.split = 1;
  c.tl.stages = 3;
  return c;
}

// The kernel a grouped call with `slots` routed slots (t * topk) launches, as
// hq_moe_gemm picks it: the choice depends on t and topk only through their
// product (slots per expert).
static bool moe_uses_smallk(const hq_plan* p, int bm) {
  return p->compute.epi == HQ_EPI_TOPK_COMBINE && p->user.kernel == 0 &&
         hq::smallk_supported(p->fmt, bm / 16, (int)(p->layer.k / 128)) && (bm == 16 || bm == 64);
}

static hq_status describe_grouped(const hq_plan* p, int64_t slots, char* buf, size_t len) {
  const MoeChoice mc = moe_choice(p, slots, 1);
  const long long n = (long long)p->layer.n, k = (long long)p->layer.k;
  if (moe_uses_smallk(p, mc.bm)) {
    snprintf(buf, len, "kernel=grouped-smallk fmt=%s slots=%lld n=%lld k=%lld experts=%d block_m=%d", fmt_name(p->fmt),
             (long long)slots, n, k, p->layer.num_experts, mc.bm);
  } else if (mc.tiled) {
    snprintf(buf, len, "kernel=grouped-tiled fmt=%s slots=%lld n=%lld k=%lld experts=%d block_m=%d tile_n=%d stages=%d",
             fmt_name(p->fmt), (long long)slots, n, k, p->layer.num_experts, mc.bm, 64 * mc.tl.nbw, mc.tl.stages);
  } else {
    snprintf(buf, len,
             "kernel=grouped-skinny fmt=%s slots=%lld n=%lld k=%lld experts=%d block_m=%d tile_n=%d waves=%d "
             "stages=%d",
             fmt_name(p->fmt), (long long)slots, n, k, p->layer.num_experts, mc.bm, 16 * mc.sk.nb, mc.sk.waves,
             mc.sk.stages);
  }
  return ok();
}

hq_status hq_moe_block_m(const hq_plan* p, int64_t t, int topk, int* block_m) {
  if (!p || !block_m) return fail(HQ_ERR_INVALID_ARG, "null argument");
  if (p->compute.kind != HQ_GEMM_GROUPED) return fail(HQ_ERR_INVALID_ARG, "not a grouped plan");
  if (t < 0 || topk < 1) return fail(HQ_ERR_INVALID_ARG, "bad sizes");
  *block_m = moe_choice(p, t, topk).bm;
  return ok();
}

hq_status hq_moe_max_padded(int64_t t, int topk, int num_experts, int block_m, int64_t* max_padded) {
  if (!max_padded) return fail(HQ_ERR_INVALID_ARG, "null argument");
  if (t < 0 || topk < 1 || num_experts < 1 || block_m < 1) return fail(HQ_ERR_INVALID_ARG, "bad sizes");
  *max_padded = moe_max_padded(t, topk, num_experts, block_m);
  return ok();
}

hq_status hq_moe_align(int64_t t, int topk, int num_experts, int block_m, const int32_t* topk_ids,
                       int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded, void* stream) {
  const hq::TimingEvents ev = hq::take_timing();  // consumed by this call whatever happens
  try {
    if (!topk_ids || !sorted_ids || !block_expert || !num_padded) return fail(HQ_ERR_INVALID_ARG, "null pointer");
    if (t < 1 || topk < 1 || num_experts < 1 || block_m < 1) return fail(HQ_ERR_INVALID_ARG, "bad sizes");
    if (t * topk > (int64_t(1) << 20)) return fail(HQ_ERR_UNSUPPORTED, "t * topk above 2^20");
    if (num_experts > 4096) return fail(HQ_ERR_UNSUPPORTED, "more than 4096 experts");
    if (block_m % 16) return fail(HQ_ERR_INVALID_ARG, "block_m must be a multiple of 16");
    hq::arm_timing(ev);
    int err = hq::launch_moe_align(t, topk, num_experts, block_m, topk_ids, sorted_ids, block_expert, num_padded,
                                   stream);
    hq::arm_timing({nullptr, nullptr});
    if (err != hipSuccess) return fail(HQ_ERR_HIP, "align launch: %s", hipGetErrorString((hipError_t)err));
    return ok();
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_moe_align");
  }
}

// Columns of N per small-K down launch.  Each launch stores its slots'
// weighted bf16 rows (t * topk * cols * 2 bytes) and the combine of the same
// columns reads them back, so the window bounds the workspace.  Windows cost
// time: each launch re-loads every block's activations and row sums (measured
// on MI355X at t = 4096, N = 7168, with fp32 rows: seven 1024-column windows
// took the down + combine from 640 to 870 us although the combine's reads
// then hit the last-level cache), so a window covers all of N up to 1 GiB of
// rows.  Equal
// windows, each a multiple of 64 columns.
static constexpr int64_t kCombineWindowBytes = int64_t(1) << 30;

static int64_t moe_down_cols(const hq_plan* p, int64_t t, int topk, int bm) {
  const int64_t N = p->layer.n;
  if (!moe_uses_smallk(p, bm) || t * topk <= 0) return N;
  int64_t c = kCombineWindowBytes / (t * topk * 2) / 64 * 64;
  if (c >= N) return N;
  c = std::max<int64_t>(c, 64);
  const int64_t n = cdiv(N, c);
  c = cdiv(cdiv(N, n), 64) * 64;
  return std::min(c, N);
}

struct MoeWs {
  size_t act32, rows, total;
};

static MoeWs moe_ws(const hq_plan* p, int64_t t, int topk) {
  MoeWs w{};
  const int64_t mp = moe_max_padded(t, topk, p->layer.num_experts, moe_choice(p, t, topk).bm);
  if (p->compute.epi == HQ_EPI_SILU_MUL_QFP8) w.act32 = align256((size_t)mp * (size_t)(p->layer.n / 2) * 4);
  if (p->compute.epi == HQ_EPI_TOPK_COMBINE)
    w.rows = align256((size_t)t * topk * (size_t)moe_down_cols(p, t, topk, moe_choice(p, t, topk).bm) * 2);
  w.total = w.act32 + w.rows;
  return w;
}

hq_status hq_moe_workspace_bytes(const hq_plan* p, int64_t t, int topk, size_t* bytes) {
  if (!p || !bytes) return fail(HQ_ERR_INVALID_ARG, "null argument");
  if (p->compute.kind != HQ_GEMM_GROUPED) return fail(HQ_ERR_INVALID_ARG, "not a grouped plan");
  if (t < 0 || t > p->max_m || topk < 1) return fail(HQ_ERR_INVALID_ARG, "t out of range [0, max_m]");
  *bytes = moe_ws(p, t, topk).total;
  return ok();
}

hq_status hq_moe_gemm(const hq_plan* p, int64_t t, int topk, const void* a, const float* a_scale,
                      const int32_t* sorted_ids, const int32_t* block_expert, const int32_t* num_padded,
                      const float* topk_w, const void* w, const void* meta, void* out, float* out_scale, void* ws,
                      size_t ws_bytes, void* stream) {
  const hq::TimingEvents ev = hq::take_timing();  // consumed by this call whatever happens
  try {
    if (!p) return fail(HQ_ERR_INVALID_ARG, "null plan");
    if (p->compute.kind != HQ_GEMM_GROUPED) return fail(HQ_ERR_INVALID_ARG, "hq_moe_gemm needs a grouped plan");
    if (t < 0 || t > p->max_m) return fail(HQ_ERR_INVALID_ARG, "t out of range [0, max_m]");
    if (topk < 1 || topk > 64) return fail(HQ_ERR_INVALID_ARG, "topk must be 1..64");
    if (t == 0) return ok();
    if (!a || !sorted_ids || !block_expert || !num_padded || !w || !meta || !out)
      return fail(HQ_ERR_INVALID_ARG, "null device pointer");
    if (!aligned16(a) || !aligned16(w) || !aligned16(meta) || !aligned16(out))
      return fail(HQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    const bool act8 = p->fmt == hq::FMT_Q8;
    if (act8 && !a_scale) return fail(HQ_ERR_INVALID_ARG, "8-bit activations need a_scale");
    if (!act8 && a_scale) return fail(HQ_ERR_INVALID_ARG, "16-bit activations take no a_scale");
    const int epi = p->compute.epi;
    if (epi == HQ_EPI_TOPK_COMBINE && !topk_w) return fail(HQ_ERR_INVALID_ARG, "the combine needs topk_w");
    if (epi == HQ_EPI_SILU_MUL_QFP8 && !out_scale) return fail(HQ_ERR_INVALID_ARG, "fp8 requant needs out_scale");
    const MoeWs mw = moe_ws(p, t, topk);
    if (mw.total > 0) {
      if (!ws) return fail(HQ_ERR_WORKSPACE, "this call needs %zu workspace bytes", mw.total);
      if (ws_bytes < mw.total) return fail(HQ_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, mw.total);
      if (!aligned16(ws)) return fail(HQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    const int64_t N = p->layer.n, K = p->layer.k, G = K / 128;
    const MoeChoice mc = moe_choice(p, t, topk);
    const int bm = mc.bm;
    const int64_t mp = moe_max_padded(t, topk, p->layer.num_experts, bm);
    {
      // the kernels address A (token rows for gate_up, aligned rows for the
      // down GEMM) and one expert's W through 32-bit buffer ranges
      const int64_t act_bytes = (p->fmt == hq::FMT_W16F16 || p->fmt == hq::FMT_W16BF16) ? 2 : 1;
      const int64_t a_rows = epi == HQ_EPI_TOPK_COMBINE ? mp : t;
      if (a_rows * K * act_bytes >= (int64_t(1) << 31) || N * K / 2 >= (int64_t(1) << 31))
        return fail(HQ_ERR_UNSUPPORTED, "activations and one expert's weights must each stay below 2 GiB");
    }
    const uint32_t* zeros = p->layer.q.zp == HQ_ZP_PER_GROUP_U4
                                ? reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(meta) +
                                                                    p->scale_region_bytes *
                                                                        (size_t)p->layer.num_experts)
                                : nullptr;
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    int mode = hq::GRP_GATHER, gepi = hq::GEPI_PLAIN;
    float* f32_out = nullptr;
    uint16_t* rows16 = nullptr;
    switch (epi) {
      case HQ_EPI_NONE: gepi = hq::GEPI_PLAIN; break;
      case HQ_EPI_SILU_MUL: gepi = hq::GEPI_SILU; break;
      case HQ_EPI_SILU_MUL_QFP8:
        gepi = hq::GEPI_SILU_F32;
        f32_out = reinterpret_cast<float*>(wsb);
        break;
      case HQ_EPI_TOPK_COMBINE:
        gepi = hq::GEPI_COMBINE;
        mode = hq::GRP_SORTED;
        rows16 = reinterpret_cast<uint16_t*>(wsb);
        break;
      default: return fail(HQ_ERR_INVALID_ARG, "unsupported grouped epilogue");
    }
    // Non-empty blocks: each holds at least one slot, so at most t * topk of
    // them exist whatever the routing; the grid covers min(that, all blocks).
    const int64_t blocks = std::min<int64_t>(mp / bm, t * topk);
    const int n_slots = (int)(t * topk);
    int err;
    const bool second = epi == HQ_EPI_SILU_MUL_QFP8 || epi == HQ_EPI_TOPK_COMBINE;
    hq::arm_timing({ev.start, second ? nullptr : ev.stop});
    // the down projection with a short K: activations resident in registers,
    // weights streamed over all columns (16- and 64-row blocks)
    const bool smallk = moe_uses_smallk(p, bm);
    if (smallk) {
      hq::SkinnyArgs s{};
      s.a = a;
      s.a_scale = a_scale;
      s.w = w;
      s.scales = meta;
      s.zeros = zeros;
      s.out = out;
      s.M = (int)mp;
      s.N = (int)N;
      s.K = (int)K;
      s.G = (int)G;
      s.gps = (int)G;
      s.zp_fixed = p->layer.q.zp == HQ_ZP_FIXED ? p->layer.q.zp_value : -1;
      s.scale_bf16 = p->layer.q.scale == HQ_BF16;
      s.out_bf16 = p->layer.q.out == HQ_BF16;
      s.sorted_ids = sorted_ids;
      s.block_expert = block_expert;
      s.num_padded = num_padded;
      s.topk_w = topk_w;
      s.topk = topk;
      s.n_slots = n_slots;
      s.epi = gepi;
      s.w_expert = (int64_t)p->w_bytes_per_expert;
      s.s_expert = (int64_t)(N * G);
      s.z_expert = (int64_t)((N / 16) * G * 2);
      s.f32_out = f32_out;
      s.rows16 = rows16;
      // column windows: down GEMM, then the combine of the same columns
      const int64_t cols = moe_down_cols(p, t, topk, bm);
      err = hipSuccess;
      for (int64_t c0 = 0; c0 < N && err == hipSuccess; c0 += cols) {
        const int64_t nc = std::min(cols, N - c0);
        s.col0 = (int)c0;
        s.ncol = (int)nc;
        hq::arm_timing({c0 == 0 ? ev.start : nullptr, nullptr});
        err = hq::launch_smallk_grouped(p->fmt, bm / 16, s, blocks, stream);
        if (err != hipSuccess) break;
        hq::arm_timing({nullptr, c0 + nc >= N ? ev.stop : nullptr});
        err = hq::launch_moe_combine(rows16, topk, t, N, c0, nc, out, p->layer.q.out == HQ_BF16, stream);
      }
      hq::arm_timing({nullptr, nullptr});
      if (err != hipSuccess) return fail(HQ_ERR_HIP, "grouped gemm launch: %s", hipGetErrorString((hipError_t)err));
      return ok();
    } else if (mc.tiled) {
      hq::TiledArgs s{};
      s.a = a;
      s.a_scale = a_scale;
      s.w = w;
      s.scales = meta;
      s.zeros = zeros;
      s.out = out;
      s.M = (int)mp;
      s.N = (int)N;
      s.K = (int)K;
      s.G = (int)G;
      s.gps = (int)G;  // grouped launches do not split K
      s.zp_fixed = p->layer.q.zp == HQ_ZP_FIXED ? p->layer.q.zp_value : -1;
      s.scale_bf16 = p->layer.q.scale == HQ_BF16;
      s.out_bf16 = p->layer.q.out == HQ_BF16;
      s.sorted_ids = sorted_ids;
      s.block_expert = block_expert;
      s.num_padded = num_padded;
      s.topk_w = topk_w;
      s.topk = topk;
      s.n_slots = n_slots;
      s.epi = gepi;
      s.half_nblk = (int)(N / 2 / 16);
      s.w_expert = (int64_t)p->w_bytes_per_expert;
      s.s_expert = (int64_t)(N * G);
      s.z_expert = (int64_t)((N / 16) * G * 2);
      s.f32_out = f32_out;
      s.rows16 = rows16;
      err = hq::launch_tiled_grouped(p->fmt, mode, mc.tl, s, blocks, stream);
    } else {
      hq::SkinnyArgs s{};
      s.a = a;
      s.a_scale = a_scale;
      s.w = w;
      s.scales = meta;
      s.zeros = zeros;
      s.out = out;
      s.M = (int)mp;
      s.N = (int)N;
      s.K = (int)K;
      s.G = (int)G;
      s.zp_fixed = p->layer.q.zp == HQ_ZP_FIXED ? p->layer.q.zp_value : -1;
      s.scale_bf16 = p->layer.q.scale == HQ_BF16;
      s.out_bf16 = p->layer.q.out == HQ_BF16;
      s.gps = (int)G;
      s.sorted_ids = sorted_ids;
      s.block_expert = block_expert;
      s.num_padded = num_padded;
      s.topk_w = topk_w;
      s.topk = topk;
      s.n_slots = n_slots;
      s.epi = gepi;
      s.half_nblk = (int)(N / 2 / 16);
      s.w_expert = (int64_t)p->w_bytes_per_expert;
      s.s_expert = (int64_t)(N * G);
      s.z_expert = (int64_t)((N / 16) * G * 2);
      s.e8_expert = (int64_t)(N * K / 32);
      s.f32_out = f32_out;
      s.rows16 = rows16;
      err = hq::launch_skinny_grouped(p->fmt, mode, mc.sk, s, blocks, stream);
    }
    hq::arm_timing({nullptr, ev.stop});
    if (err == hipSuccess && epi == HQ_EPI_SILU_MUL_QFP8)
      err = hq::launch_moe_requant(f32_out, sorted_ids, num_padded, n_slots, (int)(N / 2),
                                   std::min<int64_t>(mp, (int64_t)bm * t * topk), static_cast<uint8_t*>(out),
                                   out_scale, stream);
    if (err == hipSuccess && epi == HQ_EPI_TOPK_COMBINE)
      err = hq::launch_moe_combine(rows16, topk, t, N, 0, N, out, p->layer.q.out == HQ_BF16, stream);
    hq::arm_timing({nullptr, nullptr});
    if (err != hipSuccess) return fail(HQ_ERR_HIP, "grouped gemm launch: %s", hipGetErrorString((hipError_t)err));
    return ok();
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_moe_gemm");
  }
}

hq_status hq_moe_gemm_by_slot(const hq_plan* p, int64_t t, int topk, const void* a, const float* a_scale,
                              const int32_t* topk_ids, const float* topk_w, const void* w, const void* meta,
                              void* out, float* out_scale, void* ws, size_t ws_bytes, void* stream) {
  const hq::TimingEvents ev = hq::take_timing();  // consumed by this call whatever happens
  try {
    if (!p) return fail(HQ_ERR_INVALID_ARG, "null plan");
    if (p->compute.kind != HQ_GEMM_GROUPED) return fail(HQ_ERR_INVALID_ARG, "hq_moe_gemm_by_slot needs a grouped plan");
    if (t < 0 || t > p->max_m) return fail(HQ_ERR_INVALID_ARG, "t out of range [0, max_m]");
    if (topk < 1 || topk > 64) return fail(HQ_ERR_INVALID_ARG, "topk must be 1..64");
    if (t == 0) return ok();
    if (t * topk > 65535) return fail(HQ_ERR_UNSUPPORTED, "t * topk must be at most 65535 on this path");
    if (!a || !topk_ids || !w || !meta || !out) return fail(HQ_ERR_INVALID_ARG, "null device pointer");
    if (!aligned16(a) || !aligned16(w) || !aligned16(meta) || !aligned16(out))
      return fail(HQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    const bool act8 = p->fmt == hq::FMT_Q8;
    if (act8 && !a_scale) return fail(HQ_ERR_INVALID_ARG, "8-bit activations need a_scale");
    if (!act8 && a_scale) return fail(HQ_ERR_INVALID_ARG, "16-bit activations take no a_scale");
    const int epi = p->compute.epi;
    if (epi == HQ_EPI_TOPK_COMBINE && !topk_w) return fail(HQ_ERR_INVALID_ARG, "the combine needs topk_w");
    if (epi == HQ_EPI_SILU_MUL_QFP8 && !out_scale) return fail(HQ_ERR_INVALID_ARG, "fp8 requant needs out_scale");
    const int64_t N = p->layer.n, K = p->layer.k, G = K / 128, E = p->layer.num_experts;
    const int n_slots = (int)(t * topk);
    const bool token = epi == HQ_EPI_TOPK_COMBINE;
    const size_t need = epi == HQ_EPI_SILU_MUL_QFP8 ? align256((size_t)n_slots * (size_t)(N / 2) * 4) : 0;
    if (need > 0) {
      if (!ws) return fail(HQ_ERR_WORKSPACE, "this call needs %zu workspace bytes", need);
      if (ws_bytes < need) return fail(HQ_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, need);
      if (!aligned16(ws)) return fail(HQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    {
      // 32-bit buffer ranges: the activation rows, and one expert's weights
      // (token mode: all experts' weights and scales, the step picks one)
      const int64_t act_bytes = act8 ? 1 : 2;
      const int64_t wexp = (int64_t)p->w_bytes_per_expert;
      if ((token ? n_slots : t) * K * act_bytes >= (int64_t(1) << 31) ||
          (token ? E * wexp : wexp) >= (int64_t(1) << 31) || (token ? E * N * G * 2 : 0) >= (int64_t(1) << 31))
        return fail(HQ_ERR_UNSUPPORTED, "activations or the weights one launch addresses must stay below 2 GiB");
    }
    hq::SkinnyCfg c{};
    c.mb = 1;
    c.stages = 2;
    c.split = 1;
    {
      // defaults measured on MI355X at H = 7168, I = 256, topk 8; the plan's
      // tile_n (16, 32, 64) and waves (1..16) override them where they fit
      const hq_tuning& u = p->user;
      const bool paired = !token && (epi == HQ_EPI_SILU_MUL || epi == HQ_EPI_SILU_MUL_QFP8);
      c.nb = 2;
      if (u.tile_n == 16 || u.tile_n == 32 || u.tile_n == 64) c.nb = u.tile_n / 16;
      if (paired && c.nb < 2) c.nb = 2;
      while (c.nb > 1 && (paired ? (N / 2) % (16 * (c.nb / 2)) : N % (16 * c.nb))) c.nb /= 2;
      if (paired && c.nb < 2) return fail(HQ_ERR_UNSUPPORTED, "gate_up needs n / 2 to be a multiple of 16");
      const int64_t steps = token ? topk * G : G;
      c.waves = (u.waves >= 1 && u.waves <= 16) ? u.waves : (int)std::min<int64_t>(8, steps);
      // gate_up: 4 waves from 9 routed slots on (two alternating runs on one
      // MI355X host, the whole layer by slot at T = 4 / 8: bf16 28.7-28.9 ->
      // 28.5-28.6 and 50.0-50.3 -> 48.9-49.1 us, fp8 32.1-32.2 -> 31.4-31.6
      // and 54.5-55.2 -> 53.0-53.2 us; at T = 1, 8 waves: gate_up 8.0
      // against 9.7 us)
      if (!token && !(u.waves >= 1 && u.waves <= 16) && t * topk > 8) c.waves = 4;
      // down + combine: from 9 routed slots on, 4 column blocks of 4 waves
      // (one host, T = 4 / 8: bf16 14.4 -> 13.5 and 24.5 -> 18.6 us, fp8 15.2
      // -> 11.6 and 26.7 -> 18.0 us; at T = 1, 2 blocks of 8 waves: 5.9
      // against 9.2 us)
      if (token && t * topk > 8) {
        if (!u.tile_n && N % 64 == 0) c.nb = 4;
        if (!(u.waves >= 1 && u.waves <= 16)) c.waves = 4;
      }
    }
    const uint32_t* zeros = p->layer.q.zp == HQ_ZP_PER_GROUP_U4
                                ? reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(meta) +
                                                                    p->scale_region_bytes * (size_t)E)
                                : nullptr;
    int gepi = hq::GEPI_PLAIN;
    float* f32_out = nullptr;
    switch (epi) {
      case HQ_EPI_NONE: gepi = hq::GEPI_PLAIN; break;
      case HQ_EPI_SILU_MUL: gepi = hq::GEPI_SILU; break;
      case HQ_EPI_SILU_MUL_QFP8:
        gepi = hq::GEPI_SILU_F32;
        f32_out = static_cast<float*>(ws);
        break;
      case HQ_EPI_TOPK_COMBINE: gepi = hq::GEPI_COMBINE; break;
      default: return fail(HQ_ERR_INVALID_ARG, "unsupported grouped epilogue");
    }
    hq::SkinnyArgs s{};
    s.a = a;
    s.a_scale = a_scale;
    s.w = w;
    s.scales = meta;
    s.zeros = zeros;
    s.out = out;
    s.M = token ? (int)t : n_slots;
    s.N = (int)N;
    s.K = (int)K;
    s.G = (int)(token ? topk * G : G);  // token mode: topk slots of K / 128 groups each
    s.gps = s.G;
    s.ge = (int)G;
    s.zp_fixed = p->layer.q.zp == HQ_ZP_FIXED ? p->layer.q.zp_value : -1;
    s.scale_bf16 = p->layer.q.scale == HQ_BF16;
    s.out_bf16 = p->layer.q.out == HQ_BF16;
    s.topk_ids = topk_ids;
    s.num_experts = (int)E;
    s.topk_w = topk_w;
    s.topk = topk;
    s.n_slots = n_slots;
    s.epi = gepi;
    s.half_nblk = (int)(N / 2 / 16);
    s.w_expert = (int64_t)p->w_bytes_per_expert;
    s.s_expert = (int64_t)(N * G);
    s.z_expert = (int64_t)((N / 16) * G * 2);
    s.e8_expert = (int64_t)(N * K / 32);
    s.f32_out = f32_out;
    const bool requant = epi == HQ_EPI_SILU_MUL_QFP8;
    hq::arm_timing({ev.start, requant ? nullptr : ev.stop});
    int err = hq::launch_skinny_byslot(p->fmt, token ? hq::GRP_TOKEN : hq::GRP_SLOT, c, s, token ? t : n_slots,
                                       stream);
    hq::arm_timing({nullptr, ev.stop});
    if (err == hipSuccess && requant)
      err = hq::launch_moe_requant(f32_out, nullptr, nullptr, n_slots, (int)(N / 2), n_slots,
                                   static_cast<uint8_t*>(out), out_scale, stream);
    hq::arm_timing({nullptr, nullptr});
    if (err != hipSuccess) return fail(HQ_ERR_HIP, "grouped gemm launch: %s", hipGetErrorString((hipError_t)err));
    return ok();
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_moe_gemm_by_slot");
  }
}

hq_status hq_quantize_per_token(int64_t m, int64_t k, hq_dtype in, hq_dtype out, const void* x, void* codes,
                                float* scales, void* stream) {
  const hq::TimingEvents ev = hq::take_timing();  // consumed by this call whatever happens
  if (in != HQ_F16 && in != HQ_BF16) return fail(HQ_ERR_UNSUPPORTED, "input must be fp16 or bf16");
  if (out != HQ_FP8_E4M3 && out != HQ_INT8) return fail(HQ_ERR_UNSUPPORTED, "codes must be fp8 e4m3 or int8");
  if (m < 0 || m > (int64_t(1) << 24)) return fail(HQ_ERR_INVALID_ARG, "m out of range [0, 2^24]");
  if (k < 8 || k % 8 || k > (int64_t(1) << 24)) return fail(HQ_ERR_INVALID_ARG, "k must be a multiple of 8 in [8, 2^24]");
  if (m == 0) return ok();
  if (!x || !codes || !scales) return fail(HQ_ERR_INVALID_ARG, "null device pointer");
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
    return fail(HQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  hq::arm_timing(ev);
  const int err = hq::launch_quantize_rows(m, k, in == HQ_BF16, out == HQ_FP8_E4M3, x, codes, scales, stream);
  hq::arm_timing({nullptr, nullptr});
  if (err != hipSuccess) return fail(HQ_ERR_HIP, "quantize launch: %s", hipGetErrorString((hipError_t)err));
  return ok();
}

hq_status hq_quantize_mxfp4(int64_t m, int64_t k, hq_dtype in, const void* x, void* codes, uint8_t* e8m0,
                            void* stream) {
  const hq::TimingEvents ev = hq::take_timing();  // consumed by this call whatever happens
  if (in != HQ_F16 && in != HQ_BF16) return fail(HQ_ERR_UNSUPPORTED, "input must be fp16 or bf16");
  if (m < 0 || m > (int64_t(1) << 24)) return fail(HQ_ERR_INVALID_ARG, "m out of range [0, 2^24]");
  if (k < 128 || k % 128 || k > (int64_t(1) << 24))
    return fail(HQ_ERR_INVALID_ARG, "k must be a multiple of 128 in [128, 2^24]");
  if (m * k > (int64_t(1) << 36)) return fail(HQ_ERR_UNSUPPORTED, "m * k above 2^36");
  if (m == 0) return ok();
  if (!x || !codes || !e8m0) return fail(HQ_ERR_INVALID_ARG, "null device pointer");
  if (!aligned16(x) || !aligned16(codes) || !aligned16(e8m0))
    return fail(HQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  hq::arm_timing(ev);
  const int err = hq::launch_quantize_mx(m, k, in == HQ_BF16, x, codes, e8m0, stream);
  hq::arm_timing({nullptr, nullptr});
  if (err != hipSuccess) return fail(HQ_ERR_HIP, "quantize launch: %s", hipGetErrorString((hipError_t)err));
  return ok();
}

// ---------------------------------------------------------------------------
// autotuning (dense plans)
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

// The tuning that reproduces e through choose_exec (every field explicit).
hq_tuning resolved_tuning(const hq::Exec& e) {
  hq_tuning t{};
  if (e.kernel == hq::KER_TILED) {
    t.kernel = hq::KER_TILED;
    t.tile_m = e.tl.bm;
    t.tile_n = 64 * e.tl.nbw;
    t.waves = 4;
    t.split_k = e.tl.split;
    t.stages = e.tl.stages;
    t.tile_group = e.tl.gm;
  } else {
    t.kernel = hq::KER_SKINNY;
    t.tile_m = 16 * e.sk.mb;
    t.tile_n = 16 * e.sk.nb;
    t.waves = e.sk.waves;
    t.split_k = e.sk.split;
    t.stages = e.sk.stages;
  }
  return t;
}

bool same_tuning(const hq_tuning& a, const hq_tuning& b) {
  return a.kernel == b.kernel && a.tile_m == b.tile_m && a.tile_n == b.tile_n && a.waves == b.waves &&
         a.split_k == b.split_k && a.stages == b.stages && a.tile_group == b.tile_group;
}

// Candidate execution choices for m rows: the skinny kernel up to 64 rows
// (row / column blocks, waves, groups in flight, K split) and the tiled
// kernel from 17 rows on (tile shape, ring depth, K split).
std::vector<hq_tuning> tuning_candidates(const hq_plan* p, int64_t m) {
  std::vector<hq_tuning> c;
  if (m <= 64) {
    for (int mb : {1, 2, 4}) {
      if (mb > 1 && 16 * (mb / 2) >= m) continue;  // no tile taller than the rows need
      for (int nb : {1, 2, 4})
        for (int waves : {4, 8})
          for (int stages : {2, 4})
            for (int split : {1, 2, 4}) c.push_back(hq_tuning{hq::KER_SKINNY, 16 * mb, 16 * nb, waves, split, stages, 0, 0});
    }
  }
  if (m > 16 && p->layer.n % 128 == 0 && p->compute.epi != HQ_EPI_I32_ACC) {
    for (int bm : {64, 128})
      for (int tn : {128, 256})
        for (int stages : {2, 3, 4})
          for (int split : {1, 2, 4, 8}) c.push_back(hq_tuning{hq::KER_TILED, bm, tn, 4, split, stages, 0, 0});
  }
  return c;
}

void set_tuned(hq_plan* p, int64_t m, const hq_tuning& t) {
  for (auto& e : p->tuned)
    if (e.first == m) {
      e.second = t;
      return;
    }
  p->tuned.emplace_back(m, t);
}

}  // namespace

extern "C" {

hq_status hq_plan_set_tuning(hq_plan* p, int64_t m, const hq_tuning* t) {
  try {
    if (!p) return fail(HQ_ERR_INVALID_ARG, "null plan");
    if (p->compute.kind != HQ_GEMM_DENSE) return fail(HQ_ERR_UNSUPPORTED, "per-m tunings are for dense plans");
    if (m < 1 || m > p->max_m) return fail(HQ_ERR_INVALID_ARG, "m out of range [1, max_m]");
    if (!t) {
      for (size_t i = 0; i < p->tuned.size(); ++i)
        if (p->tuned[i].first == m) {
          p->tuned.erase(p->tuned.begin() + (long)i);
          break;
        }
      return ok();
    }
    if (t->split_k < 0 || t->split_k > 64) return fail(HQ_ERR_INVALID_ARG, "split_k must be 1..64");
    const hq::Exec e = hq::choose_exec(p, m, t);
    hq_status s = check_exec(p, e);
    if (s != HQ_OK) return s;
    set_tuned(p, m, resolved_tuning(e));
    return ok();
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_plan_set_tuning");
  }
}

hq_status hq_plan_get_tuning(const hq_plan* p, int64_t m, hq_tuning* t, int* is_tuned) {
  if (!p || !t) return fail(HQ_ERR_INVALID_ARG, "null argument");
  if (m < 1 || m > p->max_m) return fail(HQ_ERR_INVALID_ARG, "m out of range [1, max_m]");
  bool tuned = false;
  for (const auto& e : p->tuned) tuned |= e.first == m;
  *t = resolved_tuning(hq::choose_exec(p, m));
  if (is_tuned) *is_tuned = tuned ? 1 : 0;
  return ok();
}

hq_status hq_plan_set_jit(hq_plan* p, int enable, const char* cache_dir) {
  if (!p) return fail(HQ_ERR_INVALID_ARG, "null plan");
  if (enable != 0 && enable != 1) return fail(HQ_ERR_INVALID_ARG, "enable must be 0 or 1");
  if (p->compute.kind != HQ_GEMM_DENSE)
    return fail(HQ_ERR_UNSUPPORTED, "run-time specialisation covers dense plans only");
  if (cache_dir && std::strlen(cache_dir) >= sizeof(p->jit_dir))
    return fail(HQ_ERR_INVALID_ARG, "cache directory path longer than %zu bytes", sizeof(p->jit_dir) - 1);
  p->jit = enable;
  std::snprintf(p->jit_dir, sizeof(p->jit_dir), "%s", cache_dir ? cache_dir : "");
  return ok();
}

hq_status hq_jit_cache_key(const hq_plan* p, int64_t m, const char* arch, char* key, size_t key_bytes) {
  try {
    if (!p || !arch || !key) return fail(HQ_ERR_INVALID_ARG, "null argument");
    if (p->compute.kind != HQ_GEMM_DENSE)
      return fail(HQ_ERR_UNSUPPORTED, "run-time specialisation covers dense plans only");
    if (m < 1 || m > p->max_m) return fail(HQ_ERR_INVALID_ARG, "m out of range [1, max_m]");
    const hq::Exec e = hq::choose_exec(p, m);
    const int64_t N = p->layer.n, K = p->layer.k;
    const hq::jit::Spec sp = e.kernel == hq::KER_TILED ? hq::jit::tiled_spec(p->fmt, e.tl, m, N, K)
                                                        : hq::jit::skinny_spec(p->fmt, e.sk, m, N, K);
    const std::string k = hq::jit::cache_key(sp, arch);
    if (key_bytes < k.size() + 1) return fail(HQ_ERR_INVALID_ARG, "key buffer shorter than %zu bytes", k.size() + 1);
    std::memcpy(key, k.c_str(), k.size() + 1);
    return ok();
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_jit_cache_key");
  }
}

hq_status hq_jit_prepare(const hq_plan* p, int64_t m, const char* arch) {
  try {
    if (!p || !arch) return fail(HQ_ERR_INVALID_ARG, "null argument");
    if (p->compute.kind != HQ_GEMM_DENSE)
      return fail(HQ_ERR_UNSUPPORTED, "run-time specialisation covers dense plans only");
    if (m < 1 || m > p->max_m) return fail(HQ_ERR_INVALID_ARG, "m out of range [1, max_m]");
    const hq::Exec e = hq::choose_exec(p, m);
    const int64_t N = p->layer.n, K = p->layer.k;
    const hq::jit::Spec sp = e.kernel == hq::KER_TILED ? hq::jit::tiled_spec(p->fmt, e.tl, m, N, K)
                                                        : hq::jit::skinny_spec(p->fmt, e.sk, m, N, K);
    std::string err;
    const int r = hq::jit::prepare(p, sp, arch, &err);
    if (r == 1) return fail(HQ_ERR_UNSUPPORTED, "%s", err.c_str());
    if (r != 0) return fail(HQ_ERR_INTERNAL, "%s", err.c_str());
    return ok();
  } catch (...) {
    return fail(HQ_ERR_INTERNAL, "exception in hq_jit_prepare");
  }
}

hq_status hq_jit_get_stats(hq_jit_stats* stats) {
  if (!stats) return fail(HQ_ERR_INVALID_ARG, "null argument");
  const hq::jit::Stats s = hq::jit::stats();
  stats->compiles = s.compiles;
  stats->disk_hits = s.disk_hits;
  stats->memory_hits = s.memory_hits;
  stats->launches = s.launches;
  stats->compile_seconds = s.compile_seconds;
  stats->load_seconds = s.load_seconds;
  return ok();
}

hq_status hq_plan_autotune(hq_plan* p, int64_t m, const void* a, const void* a_scale, const void* w,
                           const void* meta, void* out, void* ws, size_t ws_bytes, int reps, size_t flush_bytes,
                           void* stream, hq_autotune_result* result) {
  hq::take_timing();  // an armed pair of events is not for this call
  void* flush = nullptr;
  uint32_t* sink = nullptr;
  std::vector<hipEvent_t> evs;
  auto release = [&]() {
    for (hipEvent_t e : evs) (void)hipEventDestroy(e);
    if (flush) (void)hipFree(flush);
    if (sink) (void)hipFree(sink);
  };
  try {
    if (!p) return fail(HQ_ERR_INVALID_ARG, "null plan");
    if (p->compute.kind != HQ_GEMM_DENSE) return fail(HQ_ERR_UNSUPPORTED, "autotuning is for dense plans");
    if (m < 1) return fail(HQ_ERR_INVALID_ARG, "m must be at least 1");
    if (reps < 1 || reps > 1000) return fail(HQ_ERR_INVALID_ARG, "reps must be 1..1000");
    if (flush_bytes % 16 || flush_bytes > (size_t(1) << 34))
      return fail(HQ_ERR_INVALID_ARG, "flush_bytes must be a multiple of 16, at most 16 GiB");
    hq_status s = dense_args_check(p, m, a, a_scale, w, meta, out);
    if (s != HQ_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (flush_bytes) {
      // its contents do not matter: only its reads evict the caches
      if (hipMalloc(&flush, flush_bytes) != hipSuccess || hipMalloc(reinterpret_cast<void**>(&sink), 16) != hipSuccess) {
        release();
        return fail(HQ_ERR_HIP, "cannot allocate the %zu-byte cache flush buffer", flush_bytes);
      }
    }
    evs.resize(2 * (size_t)reps, nullptr);
    for (auto& e : evs)
      if (hipEventCreate(&e) != hipSuccess) {
        e = nullptr;
        release();
        return fail(HQ_ERR_HIP, "hipEventCreate failed");
      }
    const hq::TimingEvents none{nullptr, nullptr};
    // mean time per call of one execution choice (< 0: not runnable here)
    auto time_exec = [&](const hq::Exec& e, float* us) -> hq_status {
      *us = -1.f;
      if (check_exec(p, e) != HQ_OK || e.ws_bytes > (ws ? ws_bytes : 0)) return HQ_OK;
      hq_status r = dense_run(p, e, m, a, a_scale, w, meta, out, ws, ws_bytes, stream, none);  // warm-up
      if (r != HQ_OK) return r;
      for (int i = 0; i < reps; ++i) {
        if (flush) {
          hq::arm_timing(none);
          if (hq::launch_stream_read(flush, flush_bytes, sink, 1024, stream) != hipSuccess)
            return fail(HQ_ERR_HIP, "cache flush launch failed");
        }
        if (hipEventRecord(evs[2 * i], st) != hipSuccess) return fail(HQ_ERR_HIP, "hipEventRecord failed");
        r = dense_run(p, e, m, a, a_scale, w, meta, out, ws, ws_bytes, stream, none);
        if (r != HQ_OK) return r;
        if (hipEventRecord(evs[2 * i + 1], st) != hipSuccess) return fail(HQ_ERR_HIP, "hipEventRecord failed");
      }
      if (hipEventSynchronize(evs[2 * reps - 1]) != hipSuccess) return fail(HQ_ERR_HIP, "hipEventSynchronize failed");
      double tot = 0;
      for (int i = 0; i < reps; ++i) {
        float ms = 0;
        if (hipEventElapsedTime(&ms, evs[2 * i], evs[2 * i + 1]) != hipSuccess)
          return fail(HQ_ERR_HIP, "hipEventElapsedTime failed");
        tot += ms;
      }
      *us = (float)(tot * 1000.0 / reps);
      return HQ_OK;
    };
    const hq::Exec base = hq::choose_exec(p, m);
    const hq_tuning base_t = resolved_tuning(base);
    float base_us = -1.f;
    s = time_exec(base, &base_us);
    if (s != HQ_OK) {
      release();
      return s;
    }
    if (base_us < 0) {
      release();
      return fail(HQ_ERR_WORKSPACE, "the current choice for m=%lld needs %zu workspace bytes", (long long)m,
                  base.ws_bytes);
    }
    hq_tuning best_t = base_t;
    float best_us = base_us;
    int timed = 1;
    std::vector<hq_tuning> seen{base_t};
    for (const hq_tuning& c : tuning_candidates(p, m)) {
      const hq::Exec e = hq::choose_exec(p, m, &c);
      const hq_tuning rt = resolved_tuning(e);
      bool dup = false;
      for (const auto& q : seen) dup |= same_tuning(q, rt);
      if (dup) continue;
      seen.push_back(rt);
      float us = -1.f;
      s = time_exec(e, &us);
      if (s != HQ_OK) {
        release();
        return s;
      }
      if (us < 0) continue;
      ++timed;
      if (us < best_us) {
        best_us = us;
        best_t = rt;
      }
    }
    release();
    set_tuned(p, m, best_t);
    if (result) {
      result->best = best_t;
      result->best_us = best_us;
      result->current_us = base_us;
      result->candidates = timed;
    }
    return ok();
  } catch (...) {
    release();
    return fail(HQ_ERR_INTERNAL, "exception in hq_plan_autotune");
  }
}

hq_status hq_mfma_peak(int type, int workgroups, int iters, uint32_t* sink, double* flops, void* stream) {
  if (!sink) return fail(HQ_ERR_INVALID_ARG, "null sink");
  if (type < HQ_PEAK_F16 || type > HQ_PEAK_INT8) return fail(HQ_ERR_INVALID_ARG, "unknown matrix type %d", type);
  if (workgroups < 1 || workgroups > (1 << 20)) return fail(HQ_ERR_INVALID_ARG, "workgroups out of range");
  if (iters < 1 || iters > (1 << 24)) return fail(HQ_ERR_INVALID_ARG, "iters out of range");
  if (flops) *flops = hq::mfma_peak_flops(type, workgroups, iters);
  int err = hq::launch_mfma_peak(type, workgroups, iters, sink, stream);  // takes the armed events
  hq::arm_timing({nullptr, nullptr});
  if (err != hipSuccess) return fail(HQ_ERR_HIP, "matrix probe launch: %s", hipGetErrorString((hipError_t)err));
  return ok();
}

hq_status hq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, void* stream) {
  if (!buf || !sink) return fail(HQ_ERR_INVALID_ARG, "null argument");
  if (bytes % 16 || !aligned16(buf)) return fail(HQ_ERR_INVALID_ARG, "buffer must be 16-byte aligned and sized");
  if (workgroups < 1 || workgroups > (1 << 20)) return fail(HQ_ERR_INVALID_ARG, "workgroups out of range");
  int err = hq::launch_stream_read(buf, bytes, sink, workgroups, stream);  // takes the armed events
  hq::arm_timing({nullptr, nullptr});
  if (err != hipSuccess) return fail(HQ_ERR_HIP, "stream read launch: %s", hipGetErrorString((hipError_t)err));
  return ok();
}

}  // extern "C"
