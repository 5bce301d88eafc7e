// Large-M quantized GEMM for gfx950 ("tiled" kernel): the MFMA-bound regime
// (prefill-sized M), same operation and fragment layout as the skinny kernel.
//
// Work decomposition
//   * A workgroup of 4 wavefronts computes a BM x BN output tile with
//     BN = 4 * NBW * 16: wave w owns the NBW column blocks 4*?.. of its slice
//     and all BM rows, so every weight is dequantised exactly once per tile.
//   * The k loop advances one 128-k group per iteration.  The activation tile
//     (BM rows x 128 k) is staged through LDS (double buffered, XOR-swizzled so
//     that the 16 rows read by one MFMA operand fetch hit distinct banks) and
//     shared by the 4 waves; weight fragments go from HBM straight to the
//     registers of the one wave that uses them (one 16-byte load per lane per
//     fragment).  The next group's loads are issued before the current group's
//     math, and one barrier per group separates the LDS write of group g+1
//     from the reads of group g.
//   * fp16 activations: the weights are dequantised to fp16 in registers,
//     w = ((1024 + q) - (1024 + z)) * s with packed fp16 arithmetic (the
//     subtraction is exact; one rounding in the product), and the MFMA
//     accumulates over all of K.  The other formats keep the weights as exact
//     integers in the MFMA and apply the group scale per group in fp32 (bf16:
//     with the row-sum correction of the offset 128 + z; int8: exact int32
//     per group; fp8: the row-sum correction of z), and MXFP4 feeds codes and
//     E8M0 block scales to the scaled MFMA directly.
//   * Tiles are ordered so that the workgroups the hardware places on one XCD
//     (consecutive workgroup ids modulo 8) share the same activation rows,
//     which then stay in that XCD's L2.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "hq_internal.h"

namespace hq {

template <int FMT, int BM, int NBW>
struct TCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BN = WAVES * NBW * 16;
  static constexpr int MB = BM / 16;
  static constexpr bool ACT16 = (FMT == FMT_W16F16 || FMT == FMT_W16BF16);
  static constexpr int ROWB = ACT16 ? 256 : 128;  // A bytes per row per group
  static constexpr int CHUNKS = ROWB / 16;        // 16-byte chunks per row
  static constexpr int LOADS = BM * CHUNKS / THREADS;
  static constexpr int STAGE_BYTES = BM * ROWB;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static_assert(LOADS * THREADS == BM * CHUNKS, "tile rows must fill the loaders");
};

// Physical 16-byte chunk of logical chunk c in row r (bank-conflict-free
// operand reads: the 16 rows of one MFMA operand fetch land on 16 distinct
// 16-byte bank groups).
template <bool ACT16>
__device__ inline int swz(int r, int c) {
  return ACT16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

template <int FMT, int BM, int NBW>
__global__ void __launch_bounds__(256) qgemm_tiled(TiledArgs p) {
  using C = TCfg<FMT, BM, NBW>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & 15;
  const int kq = lane >> 4;
  const int G = p.G;
  const int K = p.K;

  // XCD-aware tile order: the hardware deals workgroup ids round-robin to the
  // 8 XCDs; give the ids of one XCD consecutive logical tiles (same rows).
  const int nwg = gridDim.x;
  int lid = blockIdx.x;
  if ((nwg & 7) == 0) lid = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int tm = lid / p.tiles_n;
  const int tn = lid - tm * p.tiles_n;
  const int m0 = tm * BM;
  const int nblk0 = tn * (C::BN / 16) + wave * NBW;  // first 16-column block of this wave

  // ---- activation loader: rows / chunks this thread stages ------------------
  const uint8_t* a_bytes = static_cast<const uint8_t*>(p.a);
  const int64_t a_pitch = (int64_t)K * (C::ACT16 ? 2 : 1);
  const uint8_t* a_src[C::LOADS];
  int lds_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int idx = tid + i * C::THREADS;
    const int r = idx / C::CHUNKS;
    const int ch = idx - r * C::CHUNKS;
    const int row = min(m0 + r, p.M - 1);
    a_src[i] = a_bytes + row * a_pitch + ch * 16;
    lds_off[i] = r * C::ROWB + swz<C::ACT16>(r, ch) * 16;
  }
  u4_t a_stage[C::LOADS];
  auto load_a = [&](int g) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      a_stage[i] = *reinterpret_cast<const u4_t*>(a_src[i] + (int64_t)g * C::ROWB);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      *reinterpret_cast<u4_t*>(lds + buf * C::STAGE_BYTES + lds_off[i]) = a_stage[i];
  };

  // ---- weight fragments + group metadata of this wave -----------------------
  const u4_t* wfr = reinterpret_cast<const u4_t*>(p.w);
  u4_t braw[2][NBW];
  uint32_t sraw[2][NBW], zraw[2][NBW];
  // zero points, or (fixed zero) any readable word array of at least the same size
  const uint32_t* zsrc = p.zeros ? p.zeros : static_cast<const uint32_t*>(p.scales);
  // Loads are unconditional and decoded only in the math (no early waits).
  auto load_b = [&](auto slot_c, int g) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int64_t rec = (int64_t)(nblk0 + j) * G + g;
      braw[slot][j] = __builtin_nontemporal_load(wfr + rec * 64 + lane);
      if constexpr (FMT == FMT_F4) {
        sraw[slot][j] = p.e8m0[rec * 64 + lane];
      } else {
        sraw[slot][j] = static_cast<const uint16_t*>(p.scales)[rec * 16 + c];
        zraw[slot][j] = zsrc[rec * 2 + (c >> 3)];
      }
    }
  };
  auto zero_of = [&](uint32_t zw) -> uint32_t {
    return p.zp_fixed < 0 ? (zw >> (4 * (c & 7))) & 0xFu : (uint32_t)p.zp_fixed;
  };

  f4_t acc[C::MB][NBW];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[mb][j] = f4_t{0.f, 0.f, 0.f, 0.f};

  // Operand fetch of m-block mb from LDS stage `buf`: this lane's row
  // r = 16 mb + c.  16-bit: step t takes k = 32 t + 8 kq + [0,8) (16-byte
  // chunk 4 t + kq of the row); 8-bit: piece h takes k = 64 h + 16 kq + [0,16)
  // (chunk 4 h + kq).
  auto read_a16 = [&](int buf, int mb, u4_t (&a)[4]) {
    const int r = 16 * mb + c;
    const uint8_t* base = lds + buf * C::STAGE_BYTES + r * C::ROWB;
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const u4_t*>(base + swz<true>(r, 4 * t + kq) * 16);
  };
  auto read_a8 = [&](int buf, int mb, u4_t (&a)[2]) {
    const int r = 16 * mb + c;
    const uint8_t* base = lds + buf * C::STAGE_BYTES + r * C::ROWB;
    a[0] = *reinterpret_cast<const u4_t*>(base + swz<false>(r, kq) * 16);
    a[1] = *reinterpret_cast<const u4_t*>(base + swz<false>(r, 4 + kq) * 16);
  };

  auto compute = [&](auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int buf = slot;
    if constexpr (FMT == FMT_W16F16) {
      u4_t bop[NBW][4];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)sraw[slot][j]);
        const _Float16 cz = -(_Float16)(1024 + (int)zero_of(zraw[slot][j]));
        const h2_t s2 = h2_t{s, s};
        const h2_t c2 = h2_t{cz, cz};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u4_t x = w16_operand(braw[slot][j][t], 0x64006400u);
          uint32_t y[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            h2_t v = __builtin_bit_cast(h2_t, (uint32_t)x[r]);
            v = (v + c2) * s2;  // exact integer q - z, then one rounding
            y[r] = __builtin_bit_cast(uint32_t, v);
          }
          bop[j][t] = u4_t{y[0], y[1], y[2], y[3]};
        }
      }
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        u4_t a[4];
        read_a16(buf, mb, a);
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[mb][j] = mfma_16x16x32<true>(a[t], bop[j][t], acc[mb][j]);
      }
    } else if constexpr (FMT == FMT_W16BF16) {
      u4_t bop[NBW][4];
      float sj[NBW], cj[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        sj[j] = p.scale_bf16 ? bf16_bits_to_float(sraw[slot][j]) : f16_bits_to_float(sraw[slot][j]);
        cj[j] = 128.f + (float)zero_of(zraw[slot][j]);
#pragma unroll
        for (int t = 0; t < 4; ++t) bop[j][t] = w16_operand(braw[slot][j][t], 0x43004300u);
      }
      const u4_t ones = u4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        u4_t a[4];
        read_a16(buf, mb, a);
        f4_t rs = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) rs = mfma_16x16x32<false>(a[t], ones, rs);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          f4_t P = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) P = mfma_16x16x32<false>(a[t], bop[j][t], P);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][j][r] += sj[j] * (P[r] - cj[j] * rs[r]);
        }
      }
    } else if constexpr (FMT == FMT_I8) {
      i4_t bop[NBW][2];
      float sj[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        sj[j] = 0.0625f * (p.scale_bf16 ? bf16_bits_to_float(sraw[slot][j]) : f16_bits_to_float(sraw[slot][j]));
        bop[j][0] = i8_operand(braw[slot][j][0], braw[slot][j][1]);
        bop[j][1] = i8_operand(braw[slot][j][2], braw[slot][j][3]);
      }
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        u4_t a[2];
        read_a8(buf, mb, a);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          i4_t P = i4_t{0, 0, 0, 0};
          P = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, a[0]), bop[j][0], P, 0, 0, 0);
          P = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, a[1]), bop[j][1], P, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][j][r] += sj[j] * (float)P[r];
        }
      }
    } else if constexpr (FMT == FMT_Q8) {
      i8_t bop[NBW];
      float sj[NBW], zj[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        sj[j] = p.scale_bf16 ? bf16_bits_to_float(sraw[slot][j]) : f16_bits_to_float(sraw[slot][j]);
        zj[j] = (float)zero_of(zraw[slot][j]);
        bop[j] = q8_operand(braw[slot][j]);
      }
      const i8_t ones = i8_t{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                             0x38383838, 0x38383838, 0x38383838, 0x38383838};
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        u4_t a[2];
        read_a8(buf, mb, a);
        const i8_t av = cat8(a[0], a[1]);
        const f4_t rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, ones, f4_t{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                         0, 127, 0, 127);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const f4_t P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bop[j], f4_t{0.f, 0.f, 0.f, 0.f},
                                                                          0, 0, 0, 127, 0, 136);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][j][r] += sj[j] * (P[r] - zj[j] * rs[r]);
        }
      }
    } else {  // FMT_F4
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        u4_t a[2];
        read_a8(buf, mb, a);
        const i8_t av = cat8(a[0], a[1]);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const u4_t w = braw[slot][j];
          const i8_t bv = i8_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
          acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mb][j], 0, 4, 0, 127, 0,
                                                                        (int)sraw[slot][j]);
        }
      }
    }
  };

  // ---- main loop: one 128-k group per step, unrolled by the two buffers so
  // that every register array is indexed with compile-time constants --------
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // The next group's loads are issued without a branch (the last step
  // re-reads group G-1, which is in L2) so that the waits inside the math
  // count only LDS traffic, not the loads in flight.
  auto step = [&](auto slot_c, int g) {
    constexpr int cur = decltype(slot_c)::value;
    using Next = std::integral_constant<int, 1 - cur>;
    const int gn = min(g + 1, G - 1);
    load_a(gn);
    load_b(Next{}, gn);
    compute(slot_c);
    store_a(1 - cur);
    __syncthreads();
  };
  load_a(0);
  load_b(S0{}, 0);
  store_a(0);
  __syncthreads();
  for (int g = 0; g < G; g += 2) {
    step(S0{}, g);
    if (g + 1 < G) step(S1{}, g + 1);
  }

  // ---- epilogue ---------------------------------------------------------------
  constexpr bool ACT_SCALE = !C::ACT16;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * mb + 4 * kq + r;
      if (m >= p.M) continue;
      const float sa = ACT_SCALE ? p.a_scale[m] : 1.f;
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int n = (nblk0 + j) * 16 + c;
        store_out(p.out, (int64_t)m * p.N + n, acc[mb][j][r] * sa, p.out_bf16);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

template <int FMT, int BM, int NBW>
static hipError_t launch_tiled_t(const TiledArgs& a, hipStream_t s) {
  using C = TCfg<FMT, BM, NBW>;
  auto kern = qgemm_tiled<FMT, BM, NBW>;
  static bool attr_done = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int tiles = a.tiles_m * a.tiles_n;
  const TimingEvents ev = take_timing();
  if (ev.start)
    hipExtLaunchKernelGGL(kern, dim3(tiles), dim3(C::THREADS), (uint32_t)C::LDS_BYTES, s,
                          static_cast<hipEvent_t>(ev.start), static_cast<hipEvent_t>(ev.stop), 0, a);
  else
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(C::THREADS), C::LDS_BYTES, s, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_tiled_f(const TiledCfgRt& cfg, const TiledArgs& a, hipStream_t s) {
  if (cfg.bm == 128 && cfg.nbw == 4) return launch_tiled_t<FMT, 128, 4>(a, s);
  if (cfg.bm == 64 && cfg.nbw == 4) return launch_tiled_t<FMT, 64, 4>(a, s);
  if (cfg.bm == 128 && cfg.nbw == 2) return launch_tiled_t<FMT, 128, 2>(a, s);
  if (cfg.bm == 64 && cfg.nbw == 2) return launch_tiled_t<FMT, 64, 2>(a, s);
  return hipErrorInvalidValue;
}

int launch_tiled(int fmt, const TiledCfgRt& cfg, const TiledArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (fmt) {
    case FMT_W16F16: return (int)launch_tiled_f<FMT_W16F16>(cfg, a, s);
    case FMT_W16BF16: return (int)launch_tiled_f<FMT_W16BF16>(cfg, a, s);
    case FMT_I8: return (int)launch_tiled_f<FMT_I8>(cfg, a, s);
    case FMT_Q8: return (int)launch_tiled_f<FMT_Q8>(cfg, a, s);
    case FMT_F4: return (int)launch_tiled_f<FMT_F4>(cfg, a, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace hq
