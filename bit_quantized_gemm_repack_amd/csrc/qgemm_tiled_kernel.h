// Large-M quantized GEMM for gfx950 ("tiled" kernel): the MFMA-bound regime
// (prefill-sized M, and the grouped MoE GEMM with many tokens per expert).
// Same operation and fragment layout as the skinny kernel.
//
// Work decomposition
//   * A workgroup of 4 wavefronts computes a BM x BN output tile,
//     BN = 64 * NBW: wave w owns NBW 16-column blocks and all BM rows, so every
//     weight is dequantised exactly once per tile.
//   * The k loop advances one 128-k group per step through a 3-slot pipeline:
//       - activations (BM rows x 128 k) go from HBM straight into an LDS slot
//         with the direct global->LDS 16-byte load (no staging registers);
//         the 16-byte chunks are XOR-swizzled so that the 16 rows of one MFMA
//         operand fetch hit distinct banks;
//       - weight fragments go to a 3-slot register ring of the one wave that
//         uses them (one 16-byte load per lane per fragment), metadata beside;
//       - step g: wait until only the loads of step g+1 are still in flight,
//         one barrier (every wave's loads of step g have landed, and every
//         wave has finished reading the slot of step g-1), issue the loads of
//         step g+2 into that freed slot, then the math of step g.
//     Loads are issued without branches (past the end they re-read the last
//     group), so the number of loads in flight at every wait is exact.
//   * fp16 activations: the weights are dequantised to fp16 in registers,
//     w = ((1024 + q) - (1024 + z)) * s with packed fp16 arithmetic (the
//     subtraction is exact; one rounding in the product), and the MFMA
//     accumulates over all of K.  The other formats keep the weights as exact
//     integers in the MFMA and apply the group scale per group in fp32 (bf16:
//     with the row-sum correction of the offset 128 + z; int8: exact int32
//     per group; fp8: the row-sum correction of z), and MXFP4 feeds codes and
//     E8M0 block scales to the scaled MFMA directly.
//   * Split K (dense, for M too small to fill the chip with tiles): grid y
//     takes a contiguous range of groups and stores its fp32 partial tile
//     (times the row scale); a second kernel sums the splits in index order.
//   * Dense tiles are ordered so that the workgroups the hardware places on
//     one XCD (consecutive ids modulo 8) share the same activation rows.
//   * Grouped mode (MoE): a persistent grid of resident workgroups walks the
//     (expert-aligned block of BM slots, column tile) pairs up to the used
//     length of the aligned array; rows are gathered by token (gate_up) or
//     taken in aligned order (down); epilogues as in the skinny kernel (SiLU *
//     mul, fp32 rows for the fp8 requant, each slot's weighted bf16 row for
//     the combine kernel).
#pragma once

#ifndef __HIPCC_RTC__  // the run-time compiler takes the kernel only (hq_plan_set_jit)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#endif

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "hq_internal.h"
#ifndef __HIPCC_RTC__
#include "launch.h"
#endif

namespace hq {

template <int FMT, int BM, int NBW, int ST>
struct TCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BN = WAVES * NBW * 16;
  static constexpr int MB = BM / 16;
  static constexpr bool ACT16 = act16_fmt(FMT);
  static constexpr bool W8 = w8_weights(FMT);  // INT8 weights: two 1 KiB planes per fragment
  static constexpr bool W2 = w2_weights(FMT);  // INT2 weights: 512-byte fragments, 8 bytes per lane
  static constexpr bool W3 = w3_weights(FMT);  // INT3 weights: INT2 plane + one high-bit word per lane
  static constexpr bool TWO = W8 || W3;        // a second weight load per fragment
  static constexpr int FRAGB = frag_bytes(FMT);
  static constexpr bool ACT4 = (FMT == FMT_F44);  // MXFP4 activations
  static constexpr int ROWB = ACT16 ? 256 : (ACT4 ? 64 : 128);  // A bytes per row per group
  static constexpr int CHUNKS = ROWB / 16;        // 16-byte chunks per row
  static constexpr int RPS = 1024 / ROWB;         // rows per 1 KiB load segment
  static constexpr int NSEG = BM * ROWB / 1024;   // global->LDS loads per step (workgroup)
  static constexpr int SEGW = NSEG / WAVES;       // ... per wave
  static constexpr int STAGES = ST;  // groups in the pipeline (ST - 1 ahead of the math)
  static constexpr int STAGE_BYTES = BM * ROWB;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int META = e8m0_meta(FMT) ? 1 : 2;  // metadata loads per fragment
  // Cache policy of the weight loads: default (temporal).  The row tiles of
  // one launch-order group run side by side on one XCD and read the same
  // weight columns, so the fragments must stay in that XCD's L2.
  static constexpr int WPOL = 0;
  // vector-memory loads per step per wave (MXFP4 activations: plus one E8M0
  // word per m-block)
  static constexpr int LPS = SEGW + (TWO ? 2 : 1) * NBW + META * NBW + (ACT4 ? MB : 0);
  // the loads in flight fit the wait counter and the ring fits the LDS
  static constexpr bool FITS = ST >= 2 && LPS * (ST - 2) < 64 && LDS_BYTES <= 160 * 1024;
  static_assert(SEGW * WAVES == NSEG, "tile rows must fill the loaders");
};

// Physical 16-byte chunk of logical chunk c in row r (CH chunks per row):
// the 16 rows an MFMA operand reads at one logical chunk land on distinct
// banks.  Measured with SQ_LDS_BANK_CONFLICT on gfx950: for 64-byte rows
// (MXFP4 activations) the XOR with (r >> 1) & 3 reads without conflicts,
// where (r >> 2) & 3, r & 3 and (r ^ (r >> 2)) & 3 each cost four conflict
// cycles per 16-byte read.
template <int CH>
__device__ inline int swz(int r, int c) {
  return CH == 16 ? (c ^ (r & 15)) : (CH == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 1) & 3)));
}

// s_waitcnt: at most N (< 64) vector-memory loads of this wave still in
// flight, and every LDS read of this wave completed (so that the barrier
// that follows also orders all reads of a slot before the loads that refill it).
template <int N>
__device__ inline void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// Makes `x` look redefined here, so that no use of the value can be moved
// above this point (it pins the uses of a ring slot below the step barrier).
template <typename T>
__device__ inline void pin(T& x) {
  asm volatile("; pin %0" : "+v"(x));
}

// One BM x BN tile (row tile tm, column tile tn) of the GEMM; `lds` is the
// workgroup's stage ring.  MC, NC, KC: the call's M, N and K as compile-time
// constants (run-time specialisation, hq_plan_set_jit); 0 takes them from the
// arguments.
template <int FMT, int BM, int NBW, int GRP, int ST, int MC, int NC, int KC>
__device__ __forceinline__ void qgemm_tiled_tile(const TiledArgs& p, uint8_t* lds, int tm, int tn) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses device-only builtins; the host pass needs only the stub
  using C = TCfg<FMT, BM, NBW, ST>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int kq = lane >> 4;
  const int M = MC ? MC : p.M;
  const int N = NC ? NC : p.N;
  const int K = KC ? KC : p.K;
  const int G = KC ? KC / 128 : p.G;
  // Split K (dense only): grid y picks a range of p.gps groups; the fp32
  // partial tiles are summed by a second kernel.
  const int split = (GRP == GRP_DENSE) ? (int)blockIdx.y : 0;
  const int gb = split * p.gps;                   // first group of this split
  const int Gl = min(G - gb, p.gps);              // groups of this split (>= 1)
  const int m0 = tm * BM;

  const uint8_t* wbytes = static_cast<const uint8_t*>(p.w);
  const uint16_t* scales16 = static_cast<const uint16_t*>(p.scales);
  const uint32_t* zeros32 = p.zeros;
  const uint8_t* e8 = p.e8m0;
  [[maybe_unused]] bool paired = false;
  if constexpr (GRP != GRP_DENSE) {
    if (m0 >= *p.num_padded) return;
    const int64_t ex = p.block_expert[tm];
    if (ex < 0) {
      // slots whose expert id is out of range: no gate_up output; the down
      // GEMM writes their (weighted) slot rows as zeros for the combine
      if constexpr (GRP == GRP_SORTED) {
        for (int e = tid; e < BM * C::BN; e += C::THREADS) {
          const int r = e / C::BN, cc = e - r * C::BN;
          const int id = p.sorted_ids[m0 + r];
          if (id < p.n_slots) p.rows16[(int64_t)id * N + tn * C::BN + cc] = 0;
        }
      }
      return;
    }
    wbytes += ex * p.w_expert;
    if constexpr (e8m0_meta(FMT)) {
      e8 += ex * p.e8_expert;
    } else {
      scales16 += ex * p.s_expert;
      if (zeros32) zeros32 += ex * p.z_expert;
    }
    paired = GRP == GRP_GATHER && (p.epi == GEPI_SILU || p.epi == GEPI_SILU_F32);
  }
  // 16-column block of this wave's fragment j (gate_up pairs gate block b
  // with up block half_nblk + b: fragments j < NBW/2 gate, the rest up).
  auto nblk = [&](int j) -> int {
    if constexpr (GRP == GRP_GATHER) {
      if (paired) {
        const int b0 = tn * (C::BN / 32) + wave * (NBW / 2);
        return j < NBW / 2 ? b0 + j : p.half_nblk + b0 + (j - NBW / 2);
      }
    }
    return tn * (C::BN / 16) + wave * NBW + j;
  };

  // ---- buffer resources and this lane's byte offsets -------------------------
  // Every load goes through a buffer resource (base + byte range): the lane's
  // offset is fixed for the whole loop and the per-group advance is a scalar
  // offset, so a step spends no vector instructions on addresses.  Loads
  // outside a range return zero (the host keeps every range below 2 GiB).
  auto rsrc = [](const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
  };
  const int a_rowb = C::ACT16 ? 2 * K : (C::ACT4 ? K / 2 : K);
  const int a_rows = (GRP == GRP_GATHER) ? p.n_slots / p.topk : M;
  const auto ra = rsrc(p.a, (int64_t)a_rows * a_rowb);
  const int64_t nfrag = (int64_t)(N / 16) * G;  // fragments of this weight (one expert)
  const auto rw = rsrc(wbytes, nfrag * C::FRAGB);
  [[maybe_unused]] const auto rs = rsrc(scales16, nfrag * 32);
  [[maybe_unused]] const auto rz = rsrc(zeros32 ? static_cast<const void*>(zeros32) : static_cast<const void*>(scales16),
                                        zeros32 ? nfrag * 8 : nfrag * 32);
  [[maybe_unused]] const auto re = rsrc(e8, nfrag * byte_meta_frag(FMT));
  // MXFP4 activation scales, group-major words: word (g, row) holds the four
  // E8M0 block scales of the row's group g
  [[maybe_unused]] const auto rae = rsrc(p.a_e8m0, (int64_t)G * a_rows * 4);

  // Activation segment s (1 KiB of the slot) holds rows seg*RPS .. +RPS-1;
  // lane l writes physical chunk l % CHUNKS of row seg*RPS + l / CHUNKS, so it
  // loads the logical chunk the swizzle places there (the XOR is its own
  // inverse).
  int aoff[C::SEGW];
#pragma unroll
  for (int s = 0; s < C::SEGW; ++s) {
    const int seg = wave + C::WAVES * s;
    const int r = seg * C::RPS + lane / C::CHUNKS;
    const int lchunk = swz<C::CHUNKS>(r, lane % C::CHUNKS);
    int row;
    if constexpr (GRP == GRP_DENSE) {
      row = min(m0 + r, M - 1);
    } else if constexpr (GRP == GRP_GATHER) {
      const int id = p.sorted_ids[m0 + r];
      row = id < p.n_slots ? id / p.topk : 0;
    } else {
      row = m0 + r;
    }
    aoff[s] = row * a_rowb + lchunk * 16;
  }
  // MXFP4 activations: E8M0 word offsets of the rows 16 mb + c16 this lane's
  // MFMA operands hold (dense only); 16 rows of one m-block are 64
  // contiguous bytes
  [[maybe_unused]] int aeoff[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) aeoff[mb] = min(m0 + 16 * mb + c16, M - 1) * 4;
  int woff[NBW], soff[NBW], zoff[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int f0 = nblk(j) * G;  // first fragment of this column block
    woff[j] = f0 * C::FRAGB + lane * ((C::W2 || C::W3) ? 8 : 16);
    soff[j] = nvfp4_weights(FMT)    ? f0 * 128 + c16 * 8 + (kq >> 1) * 4
              : mxint4_weights(FMT) ? f0 * 64 + c16 * 4
                                    : (mx_weights(FMT) ? f0 * 64 + (lane & ~3) : f0 * 32 + (c16 >> 1) * 4);
    zoff[j] = f0 * 8 + (c16 >> 3) * 4;
  }

  // ---- weight fragments + metadata of this wave, register ring ---------------
  u4_t braw[C::STAGES][NBW];
  [[maybe_unused]] u4_t braw2[C::STAGES][NBW];  // INT8 weights: the low-nibble plane; INT3: the high-bit word
  uint32_t sraw[C::STAGES][NBW];
  [[maybe_unused]] uint32_t zraw[C::STAGES][NBW];
  [[maybe_unused]] uint32_t asc[C::STAGES][C::MB];  // MXFP4 activations: row scale words

  auto issue = [&](auto slot_c, int g) {
    constexpr int slot = decltype(slot_c)::value;
    const int gg = gb + g;  // uniform
#pragma unroll
    for (int s = 0; s < C::SEGW; ++s) {
      const int seg = wave + C::WAVES * s;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(lds + slot * C::STAGE_BYTES + seg * 1024), 16, aoff[s],
                                               gg * C::ROWB, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      if constexpr (C::W2 || C::W3) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rw, woff[j], gg * C::FRAGB, C::WPOL);
        braw[slot][j] = u4_t{(uint32_t)v[0], (uint32_t)v[1], 0u, 0u};
      } else {
        braw[slot][j] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[j], gg * C::FRAGB, C::WPOL));
      }
    }
    if constexpr (C::W8) {
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        braw2[slot][j] =
            __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[j] + 1024, gg * C::FRAGB, C::WPOL));
    }
    if constexpr (C::W3) {
      // the 1-bit plane: bytes [512, 768) of the fragment, one word per lane
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        braw2[slot][j] = u4_t{__builtin_amdgcn_raw_buffer_load_b32(rw, woff[j] + 512 - 4 * lane, gg * C::FRAGB, C::WPOL), 0u,
                              0u, 0u};
    }
    // Metadata comes in as whole 32-bit words and the lane's byte / half-word
    // is taken out in the math: a narrow load would be zero-extended where the
    // ring is carried round the loop, which forces a wait for every load there.
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      if constexpr (e8m0_meta(FMT)) {
        sraw[slot][j] = __builtin_amdgcn_raw_buffer_load_b32(re, soff[j], gg * byte_meta_frag(FMT), 0);
      } else {
        sraw[slot][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, soff[j], gg * 32, 0);
        zraw[slot][j] = __builtin_amdgcn_raw_buffer_load_b32(rz, zoff[j], gg * 8, 0);
      }
    }
    if constexpr (C::ACT4) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
        asc[slot][mb] = __builtin_amdgcn_raw_buffer_load_b32(rae, aeoff[mb], gg * a_rows * 4, 0);
    }
  };
  auto zero_of = [&](uint32_t zw) -> uint32_t {
    return p.zp_fixed < 0 ? (zw >> (4 * (c16 & 7))) & 0xFu : (uint32_t)p.zp_fixed;
  };
  auto scale_bits = [&](uint32_t w) -> uint32_t { return (w >> (16 * (c16 & 1))) & 0xFFFFu; };
  auto e8m0_of = [&](uint32_t w) -> int { return (int)((w >> (8 * (lane & 3))) & 0xFFu); };

  f4_t acc[C::MB][NBW];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[mb][j] = f4_t{0.f, 0.f, 0.f, 0.f};
  [[maybe_unused]] const uint32_t magic_v = opaque_vgpr(f16_act(FMT) ? 0x64006400u : 0x43004300u);
  // E8M0 block scales 2^0 and 2^9 for the scaled matrix instruction, held in
  // VGPRs: the instruction reads its scales from VGPRs only, and a uniform
  // constant left to the compiler may be placed in a scalar register.
  [[maybe_unused]] const int e8_one = (int)opaque_vgpr(127u);
  [[maybe_unused]] const int e8_nine = (int)opaque_vgpr(136u);

  // Operand fetch of m-block mb from `slot`: row r = 16 mb + c16.
  // 16-bit: step t takes k = 32 t + 8 kq + [0,8) (chunk 4 t + kq);
  // 8-bit: piece h takes k = 64 h + 16 kq + [0,16) (chunk 4 h + kq).
  auto read_a16 = [&](int slot, int mb, u4_t (&a)[4]) {
    const int r = 16 * mb + c16;
    const uint8_t* base = lds + slot * C::STAGE_BYTES + r * C::ROWB;
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const u4_t*>(base + swz<16>(r, 4 * t + kq) * 16);
  };
  auto read_a8 = [&](int slot, int mb, u4_t (&a)[2]) {
    const int r = 16 * mb + c16;
    const uint8_t* base = lds + slot * C::STAGE_BYTES + r * C::ROWB;
    a[0] = *reinterpret_cast<const u4_t*>(base + swz<8>(r, kq) * 16);
    a[1] = *reinterpret_cast<const u4_t*>(base + swz<8>(r, 4 + kq) * 16);
  };
  // 4-bit: block kq takes k = 32 kq + [0, 32) (chunk kq)
  [[maybe_unused]] auto read_a4 = [&](int slot, int mb) -> u4_t {
    const int r = 16 * mb + c16;
    const uint8_t* base = lds + slot * C::STAGE_BYTES + r * C::ROWB;
    return *reinterpret_cast<const u4_t*>(base + swz<4>(r, kq) * 16);
  };
  // 8- and 4-bit activations: the operands of every m-block of the step are
  // read into registers of their own before the first MFMA, so the LDS
  // latency is paid once per step rather than once per m-block (reading
  // into reused registers would serialise each read behind the MFMAs of the
  // m-block before).
  [[maybe_unused]] auto read_step8 = [&](int slot, u4_t (&a)[C::MB][2]) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) read_a8(slot, mb, a[mb]);
    __builtin_amdgcn_sched_barrier(0);
  };
  [[maybe_unused]] auto read_step4 = [&](int slot, u4_t (&a)[C::MB]) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) a[mb] = read_a4(slot, mb);
    __builtin_amdgcn_sched_barrier(0);
  };

  auto compute = [&](auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    if constexpr (mxint4_weights(FMT)) {
      // MXINT4: one E8M0 scale per column per MFMA step (32 k).  Per step P
      // against the offset codes OFF + (v + 8) and s_t (P - (OFF + 8)
      // rowsum_t), s_t = 2^(X_t - 127) times the element's implicit 2^-2.
      constexpr bool F16 = f16_act(FMT);
      u4_t bop[NBW][4];
      float sc[NBW][4];
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          bop[j][t] = w16_operand(braw[slot][j][t], magic_v);
          const uint32_t X = (sraw[slot][j] >> (8 * t)) & 0xFFu;
          sc[j][t] = X == 255u ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(1.0f, (int)X - 129);
        }
      const float cz = (F16 ? 1024.f : 128.f) + 8.f;
      const uint32_t one2 = F16 ? 0x3C003C00u : 0x3F803F80u;
      const u4_t ones = u4_t{one2, one2, one2, one2};
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        u4_t a[4];
        read_a16(slot, mb, a);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f4_t rs = mfma_16x16x32<F16>(a[t], ones, f4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const f4_t P = mfma_16x16x32<F16>(a[t], bop[j][t], f4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mb][j][r] += sc[j][t] * (P[r] - cz * rs[r]);
          }
        }
      }
    } else if constexpr (f16_act(FMT)) {
      // Per k-step t: the MB x NBW MFMAs of step t, with the dequantisation
      // of step t+1's weights interleaved between them (the MFMA pipe runs
      // 16 cycles per op; the 4-cycle VALU ops fill the gaps), then t+1.
      h2_t s2[NBW], c2[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)scale_bits(sraw[slot][j]));
        const _Float16 cz = -(_Float16)(1024 + (int)zero_of(zraw[slot][j]));
        s2[j] = h2_t{s, s};
        c2[j] = h2_t{cz, cz};
      }
      auto deq = [&](int j, int t) -> u4_t {
        if constexpr (nvfp4_weights(FMT)) return nvfp4_operand<false>(braw[slot][j][t], (sraw[slot][j] >> (8 * t)) & 0xFFu);
        uint32_t y[4];
        if constexpr (C::TWO) {
          // INT8: q = 16 * high + low; INT3: q = 4 * high + low;
          // (high - 0) * H + (low - z), exact integers
          const u4_t xh = C::W8 ? w16_operand(braw[slot][j][t], magic_v) : w1_operand(braw2[slot][j][0], magic_v, t);
          const u4_t xl =
              C::W8 ? w16_operand(braw2[slot][j][t], magic_v) : w2_operand(braw[slot][j][t >> 1], magic_v, t & 1);
          const h2_t m1024 = h2_t{(_Float16)-1024.f, (_Float16)-1024.f};
          const _Float16 H = (_Float16)(C::W8 ? 16.f : 4.f);
          const h2_t kh = h2_t{H, H};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const h2_t vh = __builtin_bit_cast(h2_t, (uint32_t)xh[r]) + m1024;
            const h2_t vl = __builtin_bit_cast(h2_t, (uint32_t)xl[r]) + c2[j];
            const h2_t v = (vh * kh + vl) * s2[j];  // exact integer q - z, then one rounding
            y[r] = __builtin_bit_cast(uint32_t, v);
          }
        } else {
          const u4_t x =
              C::W2 ? w2_operand(braw[slot][j][t >> 1], magic_v, t & 1) : w16_operand(braw[slot][j][t], magic_v);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            h2_t v = __builtin_bit_cast(h2_t, (uint32_t)x[r]);
            v = (v + c2[j]) * s2[j];  // exact integer q - z, then one rounding
            y[r] = __builtin_bit_cast(uint32_t, v);
          }
        }
        return u4_t{y[0], y[1], y[2], y[3]};
      };
      auto read_a16t = [&](int mb, int t) -> u4_t {
        const int r = 16 * mb + c16;
        const uint8_t* base = lds + slot * C::STAGE_BYTES + r * C::ROWB;
        return *reinterpret_cast<const u4_t*>(base + swz<16>(r, 4 * t + kq) * 16);
      };
      u4_t b[2][NBW];
      u4_t a[2][C::MB];
#pragma unroll
      for (int j = 0; j < NBW; ++j) b[0][j] = deq(j, 0);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) a[0][mb] = read_a16t(mb, 0);
      __builtin_amdgcn_sched_barrier(0);
      // One scheduling region per k-step: the next step's LDS reads first,
      // then each MFMA followed by up to three VALU ops of the next step's
      // dequantisation (the 16-cycle MFMA leaves room for three 4-cycle ops).
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int cb = t & 1, nb = cb ^ 1;
        if (t < 3) {
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) a[nb][mb] = read_a16t(mb, t + 1);
#pragma unroll
          for (int j = 0; j < NBW; ++j) b[nb][j] = deq(j, t + 1);
        }
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[mb][j] = mfma_16x16x32<true>(a[cb][mb], b[cb][j], acc[mb][j]);
        if (t < 3) __builtin_amdgcn_sched_group_barrier(0x100, C::MB, 0);
#pragma unroll
        for (int i = 0; i < C::MB * NBW; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (FMT == FMT_W8BF16 || FMT == FMT_W3BF16) {
      // INT8: q = 16 * high + low; INT3: q = 4 * high + low.  P_h and P_l
      // against (128 + high), (128 + low); the row sums remove
      // (H + 1) * 128 + z
      constexpr float kH = C::W8 ? 16.f : 4.f;
      u4_t bh[NBW][4], bl[NBW][4];
      float sj[NBW], cj[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        sj[j] = p.scale_bf16 ? bf16_bits_to_float(scale_bits(sraw[slot][j])) : f16_bits_to_float(scale_bits(sraw[slot][j]));
        cj[j] = (kH + 1.f) * 128.f + (float)zero_of(zraw[slot][j]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          bh[j][t] = C::W8 ? w16_operand(braw[slot][j][t], magic_v) : w1_operand(braw2[slot][j][0], magic_v, t);
          bl[j][t] = C::W8 ? w16_operand(braw2[slot][j][t], magic_v)
                           : w2_operand(braw[slot][j][t >> 1], magic_v, t & 1);
        }
      }
      const u4_t ones = u4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        u4_t a[4];
        read_a16(slot, mb, a);
        f4_t rs = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) rs = mfma_16x16x32<false>(a[t], ones, rs);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          f4_t Ph = f4_t{0.f, 0.f, 0.f, 0.f}, Pl = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            Ph = mfma_16x16x32<false>(a[t], bh[j][t], Ph);
            Pl = mfma_16x16x32<false>(a[t], bl[j][t], Pl);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][j][r] += sj[j] * (kH * Ph[r] + Pl[r] - cj[j] * rs[r]);
        }
      }
    } else if constexpr (FMT == FMT_NV4BF16) {
      // weights dequantised exactly in registers (nvfp4_operand), no zero point
      u4_t bop[NBW][4];
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) bop[j][t] = nvfp4_operand<true>(braw[slot][j][t], (sraw[slot][j] >> (8 * t)) & 0xFFu);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        u4_t a[4];
        read_a16(slot, mb, a);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[mb][j] = mfma_16x16x32<false>(a[t], bop[j][t], acc[mb][j]);
      }
    } else if constexpr (FMT == FMT_W16BF16 || FMT == FMT_W2BF16) {
      u4_t bop[NBW][4];
      float sj[NBW], cj[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        sj[j] = p.scale_bf16 ? bf16_bits_to_float(scale_bits(sraw[slot][j])) : f16_bits_to_float(scale_bits(sraw[slot][j]));
        cj[j] = 128.f + (float)zero_of(zraw[slot][j]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bop[j][t] = C::W2 ? w2_operand(braw[slot][j][t >> 1], magic_v, t & 1) : w16_operand(braw[slot][j][t], magic_v);
      }
      const u4_t ones = u4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
      // k-step outer over PAIR m-blocks: the PAIR (NBW + 1) accumulator chains
      // (row sums and products) advance one MFMA each per k-step, so
      // consecutive MFMAs never wait on each other's results.  Two m-blocks
      // for two column blocks per wave; with four, one m-block already has
      // five chains, and a pair would not fit the registers of two waves per
      // SIMD.
      constexpr int PAIR = (C::MB >= 2 && NBW <= 2) ? 2 : 1;
#pragma unroll
      for (int mb0 = 0; mb0 < C::MB; mb0 += PAIR) {
        u4_t a[PAIR][4];
#pragma unroll
        for (int u = 0; u < PAIR; ++u) read_a16(slot, mb0 + u, a[u]);
        f4_t rs[PAIR], P[PAIR][NBW];
#pragma unroll
        for (int u = 0; u < PAIR; ++u) {
          rs[u] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < NBW; ++j) P[u][j] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int u = 0; u < PAIR; ++u) {
            rs[u] = mfma_16x16x32<false>(a[u][t], ones, rs[u]);
#pragma unroll
            for (int j = 0; j < NBW; ++j) P[u][j] = mfma_16x16x32<false>(a[u][t], bop[j][t], P[u][j]);
          }
#pragma unroll
        for (int u = 0; u < PAIR; ++u)
#pragma unroll
          for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mb0 + u][j][r] += sj[j] * (P[u][j][r] - cj[j] * rs[u][r]);
      }
    } else if constexpr (FMT == FMT_I8) {
      i4_t bop[NBW][2];
      float sj[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        sj[j] = 0.0625f * (p.scale_bf16 ? bf16_bits_to_float(scale_bits(sraw[slot][j])) : f16_bits_to_float(scale_bits(sraw[slot][j])));
        bop[j][0] = i8_operand(braw[slot][j][0], braw[slot][j][1]);
        bop[j][1] = i8_operand(braw[slot][j][2], braw[slot][j][3]);
      }
      u4_t a8[C::MB][2];
      read_step8(slot, a8);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          i4_t P = i4_t{0, 0, 0, 0};
          P = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, a8[mb][0]), bop[j][0], P, 0, 0, 0);
          P = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, a8[mb][1]), bop[j][1], P, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][j][r] += sj[j] * (float)P[r];
        }
      }
    } else if constexpr (FMT == FMT_Q8) {
      i8_t bop[NBW];
      float sj[NBW], zj[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        sj[j] = p.scale_bf16 ? bf16_bits_to_float(scale_bits(sraw[slot][j])) : f16_bits_to_float(scale_bits(sraw[slot][j]));
        zj[j] = (float)zero_of(zraw[slot][j]);
        bop[j] = q8_operand(braw[slot][j]);
      }
      const i8_t ones = i8_t{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                             0x38383838, 0x38383838, 0x38383838, 0x38383838};
      u4_t a8[C::MB][2];
      read_step8(slot, a8);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const i8_t av = cat8(a8[mb][0], a8[mb][1]);
        const f4_t rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, ones, f4_t{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                         0, e8_one, 0, e8_one);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const f4_t P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bop[j], f4_t{0.f, 0.f, 0.f, 0.f},
                                                                          0, 0, 0, e8_one, 0, e8_nine);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][j][r] += sj[j] * (P[r] - zj[j] * rs[r]);
        }
      }
    } else if constexpr (FMT == FMT_F44) {
      // fp4 x fp4: both operands E2M1 (format 4), each with its block scales
      u4_t a4[C::MB];
      read_step4(slot, a4);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const u4_t x = a4[mb];
        const i8_t av = i8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
        const int sa = (int)((asc[slot][mb] >> (8 * kq)) & 0xFFu);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const u4_t w = braw[slot][j];
          const i8_t bv = i8_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
          acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mb][j], 4, 4, 0, sa, 0,
                                                                        e8m0_of(sraw[slot][j]));
        }
      }
    } else {  // FMT_F4
      u4_t a8[C::MB][2];
      read_step8(slot, a8);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const i8_t av = cat8(a8[mb][0], a8[mb][1]);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const u4_t w = braw[slot][j];
          const i8_t bv = i8_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
          acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mb][j], 0, 4, 0, e8_one, 0,
                                                                        e8m0_of(sraw[slot][j]));
        }
      }
    }
  };

  // ---- main loop: ST-slot pipeline, one barrier per 128-k group --------------
  auto gclamp = [&](int g) { return g < Gl ? g : Gl - 1; };
  auto step = [&](auto slot_c, int g) {
    constexpr int cur = decltype(slot_c)::value;
    using Ahead = std::integral_constant<int, (cur + ST - 1) % ST>;
    __builtin_amdgcn_sched_barrier(0);  // keeps the last step's loads above the count below
    wait_vm_lds<C::LPS * (ST - 2)>();   // this wave's loads of step g have landed (later ones may not)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      pin(braw[cur][j]);
      if constexpr (C::TWO) pin(braw2[cur][j]);
      pin(sraw[cur][j]);
      if constexpr (!e8m0_meta(FMT)) pin(zraw[cur][j]);
    }
    if constexpr (C::ACT4) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) pin(asc[cur][mb]);
    }
    issue(Ahead{}, gclamp(g + ST - 1));  // into the slot every wave finished reading at step g-1
    if (g < Gl) compute(slot_c);
  };
  // The wait count above assumes every load of a step is issued after every
  // load of the step before, so no scheduling across the prologue's steps.
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((issue(std::integral_constant<int, I>{}, gclamp(I)), __builtin_amdgcn_sched_barrier(0)), ...);
  }(std::make_integer_sequence<int, ST - 1>{});
  for (int g = 0; g < Gl; g += ST) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (step(std::integral_constant<int, I>{}, g + I), ...);
    }(std::make_integer_sequence<int, ST>{});
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS may outlive the workgroup

  // ---- epilogue ---------------------------------------------------------------
  constexpr bool ACT_SCALE = !C::ACT16 && !C::ACT4;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * mb + 4 * kq + r;
      if constexpr (GRP == GRP_DENSE) {
        if (m >= M) continue;
        const float sa = ACT_SCALE ? p.a_scale[m] : (nvfp4_weights(FMT) ? 256.f * p.tscale[0] : 1.f);
        if (p.part) {
          float* prow = p.part + ((int64_t)split * M + m) * N;
#pragma unroll
          for (int j = 0; j < NBW; ++j) prow[nblk(j) * 16 + c16] = acc[mb][j][r] * sa;
          continue;
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          store_out(p.out, (int64_t)m * N + nblk(j) * 16 + c16, acc[mb][j][r] * sa, p.out_bf16);
      } else {
        const int id = p.sorted_ids[m];
        if (id >= p.n_slots) continue;
        const int tok = id / p.topk;
        if constexpr (GRP == GRP_GATHER) {
          const float sa = ACT_SCALE ? p.a_scale[tok] : 1.f;
          if (paired) {
            const int half = N / 2;
#pragma unroll
            for (int j = 0; j < NBW / 2; ++j) {
              const float gv = acc[mb][j][r] * sa;
              const float act = gv / (1.f + expf(-gv)) * (acc[mb][j + NBW / 2][r] * sa);
              const int64_t o = (int64_t)m * half + nblk(j) * 16 + c16;
              if (p.epi == GEPI_SILU) store_out(p.out, o, act, p.out_bf16);
              else p.f32_out[o] = act;  // requantised to fp8 by moe_requant_kernel
            }
          } else {
#pragma unroll
            for (int j = 0; j < NBW; ++j)
              store_out(p.out, (int64_t)m * N + nblk(j) * 16 + c16, acc[mb][j][r] * sa, p.out_bf16);
          }
        } else {
          const float sa = (ACT_SCALE ? p.a_scale[m] : 1.f) * p.topk_w[id];
          uint16_t* row = p.rows16 + (int64_t)id * N;  // this slot's weighted row, rounded to bf16
#pragma unroll
          for (int j = 0; j < NBW; ++j) row[nblk(j) * 16 + c16] = float_to_bf16_bits(acc[mb][j][r] * sa);
        }
      }
    }
  }
#endif
}

// The kernel.  SL: the stage ring is a static LDS array (a run-time compiled
// module has no dynamic-LDS attribute to raise), not the launch's dynamic
// LDS.  Grouped 64-row tiles are held to two waves per SIMD (the persistent
// loop below must not cost the tile its occupancy).
template <int FMT, int BM, int NBW, int GRP, int ST, int MC = 0, int NC = 0, int KC = 0, int SL = 0>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((GRP != GRP_DENSE && BM == 64) ? 2 : 1)))
qgemm_tiled(TiledArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = TCfg<FMT, BM, NBW, ST>;
  static_assert(C::FITS, "loads in flight exceed the counter, or the ring the LDS");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  uint8_t* lds;
  if constexpr (SL) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_st[C::LDS_BYTES];
    lds = lds_st;
  } else {
    lds = lds_dyn;
  }
  if constexpr (GRP == GRP_DENSE) {
    // XCD-aware order: ids dealt round-robin to the 8 XCDs get consecutive
    // logical tiles on each XCD.  Logical tiles run in groups of group_m row
    // tiles, each group column by column, so the tiles one XCD holds at a time
    // form a block (group_m rows x a few columns) that shares both its
    // activation rows and its weight columns through that XCD's L2.
    const int nwg = gridDim.x;
    int lid = blockIdx.x;
    if ((nwg & 7) == 0) lid = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int per = p.group_m * p.tiles_n;  // tiles per group
    const int grp = lid / per;
    const int first = grp * p.group_m;
    const int gsz = min(p.tiles_m - first, p.group_m);
    const int r = lid - grp * per;
    qgemm_tiled_tile<FMT, BM, NBW, GRP, ST, MC, NC, KC>(p, lds, first + r % gsz, r / gsz);
  } else {
    // Grouped: persistent.  The launch holds as many workgroups as the chip
    // keeps resident (at most one per tile); each takes the (aligned block,
    // column tile) pairs blockIdx.x, blockIdx.x + gridDim.x, ... up to the
    // used length of the aligned array, read here, so that no workgroup is
    // spent on the padding the host had to allow for.  Consecutive pairs share
    // a block (one expert's weights, the same activation rows).
    const int used = min(p.tiles_m, (*p.num_padded + BM - 1) / BM);
    const int total = used * p.tiles_n;
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
      const int tm = t / p.tiles_n;
      qgemm_tiled_tile<FMT, BM, NBW, GRP, ST, MC, NC, KC>(p, lds, tm, t - tm * p.tiles_n);
      __syncthreads();  // every wave is done with the stage ring before the next tile refills it
    }
  }
#endif
}

#ifndef __HIPCC_RTC__
// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

template <int FMT, int BM, int NBW, int GRP, int ST>
inline hipError_t launch_tiled_t(const TiledArgs& a, dim3 grid, hipStream_t s) {
  using C = TCfg<FMT, BM, NBW, ST>;
  auto kern = qgemm_tiled<FMT, BM, NBW, GRP, ST>;
  static bool attr_done = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  if constexpr (GRP != GRP_DENSE) {
    // grouped launches are persistent: grid (column tiles, aligned blocks)
    // becomes as many workgroups as the chip keeps resident, at most one per
    // tile (the same count on every MI355X, so kept per instantiation)
    static int resident = 0;
    if (!resident) {
      int dev = 0, cus = 0, per = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(kern), C::THREADS,
                                                         (size_t)C::LDS_BYTES);
      if (e != hipSuccess) return e;
      resident = std::max(1, cus) * std::max(1, per);
    }
    TiledArgs b = a;
    b.tiles_n = (int)grid.x;
    b.tiles_m = (int)grid.y;
    const int64_t tiles = (int64_t)grid.x * grid.y;
    const dim3 pg((unsigned)std::min<int64_t>(tiles, resident));
    return launch_timed(kern, pg, dim3(C::THREADS), (size_t)C::LDS_BYTES, s, b);
  }
  return launch_timed(kern, grid, dim3(C::THREADS), (size_t)C::LDS_BYTES, s, a);
}

template <int FMT, int BM, int NBW, int GRP>
inline hipError_t launch_tiled_s(const TiledCfgRt& cfg, const TiledArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (GRP == GRP_DENSE) {
    if (cfg.stages == 2) return launch_tiled_t<FMT, BM, NBW, GRP, 2>(a, grid, s);
    if (cfg.stages == 4) return launch_tiled_t<FMT, BM, NBW, GRP, 4>(a, grid, s);
    if constexpr (TCfg<FMT, BM, NBW, 5>::FITS)
      if (cfg.stages == 5) return launch_tiled_t<FMT, BM, NBW, GRP, 5>(a, grid, s);
  }
  if (cfg.stages == 3 || cfg.stages == 0) return launch_tiled_t<FMT, BM, NBW, GRP, 3>(a, grid, s);
  return hipErrorInvalidValue;
}

template <int FMT, int GRP>
inline hipError_t launch_tiled_f(const TiledCfgRt& cfg, const TiledArgs& a, dim3 grid, hipStream_t s) {
  if (cfg.bm == 128 && cfg.nbw == 4) return launch_tiled_s<FMT, 128, 4, GRP>(cfg, a, grid, s);
  if (cfg.bm == 64 && cfg.nbw == 4) return launch_tiled_s<FMT, 64, 4, GRP>(cfg, a, grid, s);
  if (cfg.bm == 128 && cfg.nbw == 2) return launch_tiled_s<FMT, 128, 2, GRP>(cfg, a, grid, s);
  if (cfg.bm == 64 && cfg.nbw == 2) return launch_tiled_s<FMT, 64, 2, GRP>(cfg, a, grid, s);
  return hipErrorInvalidValue;
}

// Every split must hold at least one group: the kernel's loads clamp group
// indices into [first group of the split, last group of the split].
inline bool splits_cover_k(const TiledCfgRt& cfg, const TiledArgs& a, bool dense) {
  const int splits = (dense && a.part) ? cfg.split : 1;
  return a.G >= 1 && a.gps >= 1 && (int64_t)(splits - 1) * a.gps < a.G && (int64_t)splits * a.gps >= a.G;
}

// The fp16-activation instantiations live in a translation unit of their own
// (built with matrix-instruction results in accumulation registers, which
// their epilogue-free k loop prefers); the other formats are built with the
// results in ordinary VGPRs, which their per-group epilogues read.
hipError_t launch_tiled_f16(int fmt, int mode, const TiledCfgRt& cfg, const TiledArgs& a, dim3 grid, hipStream_t s);

#endif  // __HIPCC_RTC__

}  // namespace hq
