// Grouped GEMM for a short reduction (K = 128 G, G <= 4): the MoE down
// projection with its top-k combine rows (Humming page on news.ditty.ir,
// summary: the grouped MoE path; cocoloop.cn speed-up table, MoE row).
//
// The down GEMM of one GPU's share of the layer has K = 256 (two groups) and
// N = 7168: the reduction is too short for a K-split or a K-pipelined tile to
// amortise its start-up, and the output (one row per routed slot) is larger
// than the weights.  So here
//   * a workgroup takes one expert-aligned block of 16 MB rows and a chunk of
//     the columns; each of its 4 waves holds the block's activation operands
//     for the whole of K in registers (loaded once), together with the row
//     sums of every group;
//   * each wave then walks its column blocks (16 columns each, interleaved
//     over the waves), streaming the G weight fragments of a block with D
//     blocks of loads in flight (branch-free, so the waits are partial);
//   * per column block the MFMA sees the exact integer codes (OFF + q) and the
//     group scale and zero point are applied in fp32 with the row sums:
//       o[m, n] = sum_g s[n,g] (P_g[m,n] - (OFF + z[n,g]) rowsum_g(a[m, :]))
//     (fp8 activations: OFF = 0, codes q * 2^-9 undone by the MFMA's block
//     scale, times the row scale);
//   * the epilogue stores topk_w * o, rounded to bf16, as the slot's row for
//     the combine (half the traffic of fp32 rows, which at 32k routed slots
//     outweigh every other operand of the layer).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "hq_internal.h"
#include "launch.h"

namespace hq {

template <int FMT, int MB, int G, int D>
__global__ void __launch_bounds__(256) qgemm_smallk(SkinnyArgs p) {
  constexpr bool ACT16 = (FMT == FMT_W16F16 || FMT == FMT_W16BF16);
  constexpr int AV = ACT16 ? 4 * G : 2 * G;  // 16-byte activation operands per m-block
  const int lane = threadIdx.x & 63;
  // E8M0 block scales 2^0 and 2^9 for the scaled matrix instruction, held in
  // VGPRs: the instruction reads its scales from VGPRs only, and a uniform
  // constant left to the compiler may be placed in a scalar register.
  [[maybe_unused]] const int e8_one = (int)opaque_vgpr(127u);
  [[maybe_unused]] const int e8_nine = (int)opaque_vgpr(136u);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar column offsets
  const int c = lane & 15;
  const int kq = lane >> 4;
  const int b = blockIdx.y;
  const int m0 = b * 16 * MB;
  if (m0 >= *p.num_padded) return;
  // this launch's column window: blocks [cbase, cbase + nblocks) of N; slot
  // rows are stored window-local, [n_slots][ncol]
  const int ncol = p.ncol ? p.ncol : p.N;
  const int cbase = p.col0 / 16;
  const int nblocks = ncol / 16;
  const int per_chunk = (nblocks + gridDim.x - 1) / gridDim.x;
  const int cb0 = blockIdx.x * per_chunk;
  const int cb1 = min(nblocks, cb0 + per_chunk);
  if (cb0 >= cb1) return;
  const int64_t ex = p.block_expert[b];
  if (ex < 0) {
    // slots whose expert id is out of range: zero rows for the combine
    for (int e = threadIdx.x; e < 16 * MB * (cb1 - cb0) * 16; e += blockDim.x) {
      const int r = e / ((cb1 - cb0) * 16), cc = e - r * ((cb1 - cb0) * 16);
      const int id = p.sorted_ids[m0 + r];
      if (id < p.n_slots) p.rows16[(int64_t)id * ncol + cb0 * 16 + cc] = 0;
    }
    return;
  }
  const u4_t* wfr = reinterpret_cast<const u4_t*>(static_cast<const uint8_t*>(p.w) + ex * p.w_expert);
  const uint16_t* scales16 = static_cast<const uint16_t*>(p.scales) + ex * p.s_expert;
  const uint32_t* zsrc = p.zeros ? p.zeros + ex * p.z_expert : reinterpret_cast<const uint32_t*>(scales16);
  const int K = p.K;

  // output rows of this lane: slot ids, weights (topk_w times the row scale)
  // and the byte offset of (row, column c) in the window's slot rows; a
  // padding row gets an offset past the buffer range, so its stores are
  // dropped by the range check instead of a branch.  The rows of one window
  // stay below 2 GiB (the host caps a window at 1 GiB).
  int oid[MB][4];
  float of[MB][4];
  int ooff[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * mb + 4 * kq + r;
      const int id = p.sorted_ids[m];
      oid[mb][r] = id;
      of[mb][r] = id < p.n_slots ? p.topk_w[id] * (ACT16 ? 1.f : p.a_scale[m]) : 0.f;
      ooff[mb][r] = id < p.n_slots ? (id * ncol + c) * 2 : INT32_MIN;
    }
  const auto rout = __builtin_amdgcn_make_buffer_rsrc(p.rows16, (short)0, (int)((int64_t)p.n_slots * ncol * 2),
                                                      0x00020000);
  // m-blocks up to the last one that holds a slot (an expert's slots come
  // first in its aligned segment, so a block's padding rows usually fill its
  // last m-blocks): the others need no operands, products or stores
  uint32_t live = 0;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    bool any = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) any |= oid[mb][r] < p.n_slots;
    if (__builtin_amdgcn_ballot_w64(any) != 0) live |= 1u << mb;
  }
  const int nlive = live ? 32 - __builtin_clz(live) : 0;

  // ---- the block's activation operands and row sums, once ----------------
  // 16-bit step t of group g: k = 128 g + 32 t + 8 kq + [0,8); 8-bit piece h:
  // k = 128 g + 64 h + 16 kq + [0,16).
  u4_t a[MB][AV];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= nlive) break;
    const int64_t row = m0 + 16 * mb + c;  // aligned rows: the down GEMM's input rows
    if constexpr (ACT16) {
      const uint16_t* ar = static_cast<const uint16_t*>(p.a) + row * K + 8 * kq;
#pragma unroll
      for (int v = 0; v < AV; ++v) a[mb][v] = *reinterpret_cast<const u4_t*>(ar + (v / 4) * 128 + 32 * (v % 4));
    } else {
      const uint8_t* ar = static_cast<const uint8_t*>(p.a) + row * K + 16 * kq;
#pragma unroll
      for (int v = 0; v < AV; ++v) a[mb][v] = *reinterpret_cast<const u4_t*>(ar + (v / 2) * 128 + 64 * (v % 2));
    }
  }
  f4_t rs[MB][G];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= nlive) break;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if constexpr (ACT16) {
        const uint32_t one2 = (FMT == FMT_W16F16) ? 0x3C003C00u : 0x3F803F80u;
        const u4_t ones = u4_t{one2, one2, one2, one2};
        f4_t s = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) s = mfma_16x16x32<FMT == FMT_W16F16>(a[mb][4 * g + t], ones, s);
        rs[mb][g] = s;
      } else {
        const i8_t ones = i8_t{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                               0x38383838, 0x38383838, 0x38383838, 0x38383838};
        rs[mb][g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            cat8(a[mb][2 * g], a[mb][2 * g + 1]), ones, f4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, e8_one, 0, e8_one);
      }
    }
  }

  // ---- column blocks of this wave, D blocks of loads in flight ------------
  const int n_my = (cb1 - cb0 - wave + 3) / 4;  // blocks cb0 + wave + 4 i
  const int cb_last = cb1 - 1;
  struct St {
    u4_t w[G];
    uint32_t s[G];
    uint32_t z[G];
  };
  auto cb_of = [&](int i) { return i < n_my ? cb0 + wave + 4 * i : cb_last; };
  auto load = [&](St& st, int cbl) {
    const int64_t cb = cbase + cbl;  // column block of N
#pragma unroll
    for (int g = 0; g < G; ++g) st.w[g] = __builtin_nontemporal_load(wfr + (cb * G + g) * 64 + lane);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t rec = cb * G + g;
      st.s[g] = reinterpret_cast<const uint32_t*>(scales16)[(rec * 16 + c) >> 1];
      st.z[g] = zsrc[rec * 2 + (c >> 3)];
    }
  };
  // the 16-bit operands' exponent pattern in a VGPR: one v_and_or_b32 per
  // unpacked register (mask literal, magic register)
  [[maybe_unused]] const uint32_t magic_v = opaque_vgpr((FMT == FMT_W16F16) ? 0x64006400u : 0x43004300u);
  auto compute = [&](auto L_c, const St& st, int cb) {
    constexpr int L = decltype(L_c)::value;  // live m-blocks
    f4_t acc[L];
#pragma unroll
    for (int mb = 0; mb < L; ++mb) acc[mb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint32_t sb = (st.s[g] >> (16 * (c & 1))) & 0xFFFFu;
      const float s = p.scale_bf16 ? bf16_bits_to_float(sb) : f16_bits_to_float(sb);
      const uint32_t z = p.zp_fixed < 0 ? (st.z[g] >> (4 * (c & 7))) & 0xFu : (uint32_t)p.zp_fixed;
      if constexpr (ACT16) {
        const uint32_t magic = magic_v;
        const float cz = ((FMT == FMT_W16F16) ? 1024.f : 128.f) + (float)z;
        f4_t P[L];
#pragma unroll
        for (int mb = 0; mb < L; ++mb) P[mb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u4_t bop = w16_operand(st.w[g][t], magic);
#pragma unroll
          for (int mb = 0; mb < L; ++mb) P[mb] = mfma_16x16x32<FMT == FMT_W16F16>(a[mb][4 * g + t], bop, P[mb]);
        }
#pragma unroll
        for (int mb = 0; mb < L; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][r] += s * (P[mb][r] - cz * rs[mb][g][r]);
      } else {
        const i8_t bop = q8_operand(st.w[g]);
        const float zf = (float)z;
#pragma unroll
        for (int mb = 0; mb < L; ++mb) {
          // codes 0x00..0x0F are q * 2^-9 in e4m3; block scale 2^9 (E8M0 136) undoes it
          const f4_t P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              cat8(a[mb][2 * g], a[mb][2 * g + 1]), bop, f4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, e8_one, 0, e8_nine);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][r] += s * (P[r] - zf * rs[mb][g][r]);
        }
      }
    }
    // column block cb of the window: a scalar byte offset on every row
#pragma unroll
    for (int mb = 0; mb < L; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)float_to_bf16_bits(acc[mb][r] * of[mb][r]), rout, ooff[mb][r],
                                              cb * 32, 0);
  };
  auto run = [&](auto L_c) {
    St st[D];
#pragma unroll
    for (int d = 0; d < D; ++d) load(st[d], cb_of(d));
    for (int i = 0; i < n_my; i += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (i + d < n_my) compute(L_c, st[d], cb0 + wave + 4 * (i + d));
        load(st[d], cb_of(i + d + D));
      }
    }
  };
  if constexpr (MB == 4) {
    if (nlive <= 1) run(std::integral_constant<int, 1>{});
    else if (nlive == 2) run(std::integral_constant<int, 2>{});
    else if (nlive == 3) run(std::integral_constant<int, 3>{});
    else run(std::integral_constant<int, 4>{});
  } else {
    run(std::integral_constant<int, MB>{});
  }
}

template <int FMT, int MB, int G>
static hipError_t launch_smallk_t(const SkinnyArgs& a, dim3 grid, hipStream_t s) {
  return launch_timed(qgemm_smallk<FMT, MB, G, 4>, grid, dim3(256), 0, s, a);
}

template <int FMT>
static hipError_t launch_smallk_f(int mb, const SkinnyArgs& a, dim3 grid, hipStream_t s) {
  if (mb == 1 && a.G == 1) return launch_smallk_t<FMT, 1, 1>(a, grid, s);
  if (mb == 1 && a.G == 2) return launch_smallk_t<FMT, 1, 2>(a, grid, s);
  if (mb == 1 && a.G == 4) return launch_smallk_t<FMT, 1, 4>(a, grid, s);
  if (mb == 4 && a.G == 1) return launch_smallk_t<FMT, 4, 1>(a, grid, s);
  if (mb == 4 && a.G == 2) return launch_smallk_t<FMT, 4, 2>(a, grid, s);
  return hipErrorInvalidValue;
}

bool smallk_supported(int fmt, int mb, int G) {
  if (fmt != FMT_W16F16 && fmt != FMT_W16BF16 && fmt != FMT_Q8) return false;
  return (mb == 1 && (G == 1 || G == 2 || G == 4)) || (mb == 4 && (G == 1 || G == 2));
}

int launch_smallk_grouped(int fmt, int mb, const SkinnyArgs& a, int64_t blocks, void* stream) {
  const int ncol = a.ncol ? a.ncol : a.N;
  if (!smallk_supported(fmt, mb, a.G) || a.epi != GEPI_COMBINE || a.N % 16 || a.K != 128 * a.G || ncol % 16 ||
      a.col0 % 16 || a.col0 < 0 || a.col0 + ncol > a.N)
    return (int)hipErrorInvalidValue;
  // column chunks of the window: about 1024 workgroups per launch, at least
  // one column block per wave
  const int64_t nblocks = ncol / 16;
  int64_t chunks = (1024 + blocks - 1) / blocks;
  chunks = std::max<int64_t>(1, std::min<int64_t>(chunks, nblocks / 4));
  const dim3 grid((unsigned)chunks, (unsigned)blocks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (fmt) {
    case FMT_W16F16: return (int)launch_smallk_f<FMT_W16F16>(mb, a, grid, s);
    case FMT_W16BF16: return (int)launch_smallk_f<FMT_W16BF16>(mb, a, grid, s);
    case FMT_Q8: return (int)launch_smallk_f<FMT_Q8>(mb, a, grid, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace hq
