// Small-M quantized GEMM for gfx950 ("skinny" kernel): the weight-bandwidth
// bound regime (decode, M <= 64 per launch slice).
//
// Operation (Humming page on news.ditty.ir, summary: weights, scales and zero
// points are separate parameters; W4A16 and W4A8 including MXFP4 x FP8):
//   C[m,n] = s_a[m] * sum_g s[n,g] * sum_{k in g} a[m,k] * (q[n,k] - z[n,g])
// or, for MXFP4, C[m,n] = s_a[m] * sum_k a[m,k] * e2m1(q[n,k]) * 2^(X[n,k/32]-127).
//
// Work decomposition
//   * A workgroup owns NB blocks of 16 output columns and MB blocks of 16 rows
//     and a contiguous range of 128-k groups (its split).  Its W wavefronts
//     take the groups of that range round-robin, so at any time the waves of a
//     workgroup stream neighbouring 1 KiB weight fragments.
//   * Weights go straight from HBM to registers with one 16-byte load per
//     lane per fragment (fully coalesced, no LDS: no other wave needs them).
//     Each wave keeps STAGES groups of loads in flight ahead of its math.
//   * Activations are read per lane as one contiguous 32 / 64-byte run of a
//     row (L2 / L1 resident; rows beyond M are clamped, their results dropped).
//     Dense 16-bit activations of a few rows, and a routed slot's token row
//     in slot mode, may instead be copied once into LDS (AS = 1: the block's
//     rows over its split's K range, while the first weight loads are in
//     flight) and read from there: per group, four 64-lane
//     global loads of which only the lanes of rows below M carry data would
//     otherwise take as much address-unit time as the weight loads.
//   * Per group the 4-bit codes become MFMA operands with one mask (+ one
//     shift) per register and no float arithmetic: the MFMA sees the exact
//     integers (OFF + q) (16-bit formats: OFF = 1024 for fp16, 128 for bf16),
//     q (fp8, via the e4m3 codes 0x00..0x0F = q * 2^-9, undone by the MFMA's
//     block scale 2^9) or 16 (q - 8) (int8).  The zero point and the offset
//     are removed with the row sums of A over the group, obtained from one
//     extra MFMA chain against a ones operand (shared by all column blocks):
//       acc += s[n,g] * (P[m,n,g] - (OFF + z[n,g]) * rowsum_g(a[m, :]))
//     so the group scale is applied once per output in fp32 and the weights
//     are never rounded.  MXFP4 needs no conversion at all: its codes and
//     E8M0 scales feed the scaled MFMA directly.
//   * The W partial accumulators are summed in LDS in a fixed order; with a
//     split > 1 every workgroup stores its fp32 partial tile (times the row
//     scale) and a second kernel sums the splits in index order.  Results are
//     therefore deterministic run to run.
#pragma once

#ifndef __HIPCC_RTC__  // the run-time compiler takes the kernel only (hq_plan_set_jit)
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#endif

#include "device_common.h"
#include "hq_internal.h"

namespace hq {

template <int FMT>
struct FmtInfo {
  static constexpr bool kAct16 = act16_fmt(FMT);
  static constexpr bool kW8 = w8_weights(FMT);  // INT8 weights: a second (low-nibble) plane
  static constexpr bool kW2 = w2_weights(FMT);  // INT2 weights: 8 bytes per lane per fragment
  static constexpr bool kW3 = w3_weights(FMT);  // INT3 weights: INT2 plane (8 B) + 1-bit plane (4 B) per lane
  static constexpr bool kMX4 = mxint4_weights(FMT);  // MXINT4: one E8M0 scale per column per MFMA step
  static constexpr bool kNV4 = nvfp4_weights(FMT);   // NVFP4: E4M3 per 16 k, dequantised in registers
  static constexpr bool kAct4 = (FMT == FMT_F44);  // MXFP4 activations
  static constexpr int kAVec = kAct16 ? 4 : (kAct4 ? 1 : 2);  // 16-byte loads per lane per group
  static constexpr int kARowB = kAct16 ? 256 : (kAct4 ? 64 : 128);  // A bytes per row per group
  static constexpr bool kRowSum = (act16_fmt(FMT) || FMT == FMT_Q8);
  static constexpr bool kActScale = !kAct16 && !kAct4;  // one fp32 scale per row
};

template <int FMT, int MB, int NB>
struct Stage {
  u4_t a[MB][FmtInfo<FMT>::kAVec];
  u4_t b[NB];
  u4_t b2[NB];        // INT8 weights: the low-nibble plane (b holds the high one); INT3: the high-bit word
  uint32_t sraw[NB];  // scale bits, or the E8M0 byte
  uint32_t zraw[NB];  // zero-point word (8 nibbles), unused with a fixed zero
  uint32_t asc[MB];   // MXFP4 activations: the row's four E8M0 block scales of the group
  float gw;           // token mode: the step's top-k weight (times its slot row's scale)
};

// s_waitcnt: at most N (< 64) vector-memory loads of this wave in flight
// (LDS and scalar counters not waited on).
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int FMT>
__device__ inline f4_t mfma16(u4_t a, u4_t b, f4_t c) {
  return mfma_16x16x32<f16_act(FMT)>(a, b, c);
}

// GRP selects the row / weight indexing: GRP_DENSE (rows 0..M-1, one weight),
// GRP_GATHER (MoE gate_up: block z of the expert-aligned slot array, rows are
// the slots' tokens, weights of the block's expert), GRP_SORTED (MoE down:
// rows are the aligned slots themselves), GRP_SLOT (gate_up without the
// alignment: block z is routed slot z, one row, its token's activations
// against its expert's weights, output row z) or GRP_TOKEN (down and combine
// in one: block z is token z and its k loop runs over the token's topk slots
// in turn, each slot's activation row against that slot's expert, the top-k
// weight folded into the group scale, so the row sum is the combined output).
// MC, NC, KC: the call's M, N and K as compile-time constants (run-time
// specialisation, hq_plan_set_jit); 0 takes them from the arguments.  SL:
// the reduction buffer is a static LDS array sized for MAXT threads (a
// run-time compiled module has no dynamic-LDS attribute to raise), not the
// launch's dynamic LDS.  AS: the activation slab is staged in LDS behind the
// reduction buffer (16-bit activations, one row block, dense or slot mode;
// a_pitch > 0).
template <int FMT, int MB, int NB, int STAGES, int MAXT, int GRP, int MC = 0, int NC = 0, int KC = 0, int SL = 0,
          int AS = 0>
__global__ void __launch_bounds__(MAXT) qgemm_skinny(SkinnyArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses device-only builtins; the host pass needs only the stub
  using FI = FmtInfo<FMT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar group offsets
  const int W = blockDim.x >> 6;
  const int c = lane & 15;
  const int kq = lane >> 4;
  const int nt = blockIdx.x;
  const int split = blockIdx.y;
  const int m0 = blockIdx.z * 16 * MB;
  const int M = MC ? MC : p.M;
  const int N = NC ? NC : p.N;
  const int K = KC ? KC : p.K;
  const int G = KC ? KC / 128 : p.G;

  // Grouped mode: skip blocks past the aligned length; point at this block's
  // expert.  gate_up pairs gate column block j with up column block
  // half_nblk + j inside one workgroup (first NB/2 blocks gate, rest up).
  const uint8_t* wbytes = static_cast<const uint8_t*>(p.w);
  const uint16_t* scales16 = static_cast<const uint16_t*>(p.scales);
  const uint32_t* zeros32 = p.zeros;
  const uint8_t* e8 = p.e8m0;
  [[maybe_unused]] bool paired = false;
  if constexpr (GRP == GRP_SLOT) {
    // one routed slot per block: its expert straight from the routing
    const int slot = blockIdx.z;
    const int ex = p.topk_ids[slot];
    paired = p.epi == GEPI_SILU || p.epi == GEPI_SILU_F32;
    if (ex < 0 || ex >= p.num_experts) {
      // out-of-range expert: a zero output row (the token-mode down weights it by zero)
      const int width = paired ? N / 2 : N, cols = (paired ? NB / 2 : NB) * 16;
      for (int e = threadIdx.x; e < cols; e += blockDim.x) {
        const int64_t o = (int64_t)slot * width + nt * cols + e;
        if (p.epi == GEPI_SILU_F32) p.f32_out[o] = 0.f;
        else store_out(p.out, o, 0.f, p.out_bf16);
      }
      return;
    }
    wbytes += (int64_t)ex * p.w_expert;
    if constexpr (e8m0_meta(FMT)) {
      e8 += (int64_t)ex * p.e8_expert;
    } else {
      scales16 += (int64_t)ex * p.s_expert;
      if (zeros32) zeros32 += (int64_t)ex * p.z_expert;
    }
  } else if constexpr (GRP == GRP_TOKEN) {
    // the expert changes along k: addressed per step (below); 16-bit scales only
    static_assert(!e8m0_meta(FMT), "token mode takes formats with 16-bit group scales");
  } else if constexpr (GRP != GRP_DENSE) {
    if (m0 >= *p.num_padded) return;
    const int64_t ex = p.block_expert[blockIdx.z];
    if (ex < 0) {
      // slots whose expert id is out of range: no gate_up output; the down
      // GEMM writes their (weighted) slot rows as zeros for the combine
      if constexpr (GRP == GRP_SORTED) {
        for (int e = threadIdx.x; e < 16 * MB * NB * 16; e += blockDim.x) {
          const int r = e / (NB * 16), cc = e - r * (NB * 16);
          const int id = p.sorted_ids[m0 + r];
          if (id < p.n_slots) p.rows16[(int64_t)id * N + (nt * NB + cc / 16) * 16 + (cc & 15)] = 0;
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
  auto nblk = [&](int nb) -> int {
    if constexpr (GRP == GRP_GATHER || GRP == GRP_SLOT) {
      if (paired) return nb < NB / 2 ? nt * (NB / 2) + nb : p.half_nblk + nt * (NB / 2) + (nb - NB / 2);
    }
    return nt * NB + nb;
  };

  const int g_beg = split * p.gps;
  const int g_end = min(G, g_beg + p.gps);
  const int my_first = g_beg + wave;
  const int n_it = (my_first < g_end) ? (g_end - my_first + W - 1) / W : 0;

  // ---- buffer resources and this lane's byte offsets -------------------------
  // Every load goes through a buffer resource: the lane's offset is fixed and
  // the group advance is a scalar offset.  A lane whose row holds no output
  // (past M, or a padding slot) gets an offset outside the activation range:
  // the load returns zero without touching memory, so the activation loads of
  // a 1..15-row block fetch only the rows that exist.
  auto rsrc = [](const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
  };
  const int a_rowb = FI::kAct16 ? 2 * K : (FI::kAct4 ? K / 2 : K);
  // activation rows: tokens (gate_up modes), slot rows (token mode), else M
  const int a_rows = (GRP == GRP_GATHER || GRP == GRP_SLOT) ? p.n_slots / p.topk
                                                            : (GRP == GRP_TOKEN ? p.n_slots : M);
  const auto ra = rsrc(p.a, (int64_t)a_rows * a_rowb);
  const int GW = GRP == GRP_TOKEN ? p.ge : G;  // groups of one expert's weight
  const int64_t nfrag = (int64_t)(N / 16) * GW;
  constexpr int kFragB = frag_bytes(FMT);  // weight bytes per 16 x 128 fragment
  // token mode reads every expert's layout (the step picks one): ranges over all of them
  const int64_t n_exp = GRP == GRP_TOKEN ? p.num_experts : 1;
  const auto rw = rsrc(wbytes, GRP == GRP_TOKEN ? n_exp * p.w_expert : nfrag * kFragB);
  [[maybe_unused]] const auto rsc = rsrc(scales16, GRP == GRP_TOKEN ? n_exp * p.s_expert * 2 : nfrag * 32);
  [[maybe_unused]] const auto rz = rsrc(zeros32 ? static_cast<const void*>(zeros32) : static_cast<const void*>(scales16),
                                        zeros32 ? (GRP == GRP_TOKEN ? n_exp * p.z_expert * 4 : nfrag * 8)
                                                : (GRP == GRP_TOKEN ? n_exp * p.s_expert * 2 : nfrag * 32));
  [[maybe_unused]] const auto re = rsrc(e8, nfrag * byte_meta_frag(FMT));
  // NVFP4: the operands carry e2m1 * e4m3 * 2^-8; the epilogue applies 2^8 and the tensor scale
  [[maybe_unused]] const float nv_scale = FI::kNV4 ? 256.f * p.tscale[0] : 1.f;
  // MXFP4 activation scales, group-major words: word (g, row) holds the four
  // E8M0 block scales of the row's group g
  [[maybe_unused]] const auto rae = rsrc(p.a_e8m0, (int64_t)G * a_rows * 4);
  // Staged activations (AS): the block's rows over this split's groups sit in
  // LDS behind the reduction buffer, row r at r * a_pitch, group g at
  // (g - g_beg) * 256 bytes.
  static_assert(!AS || ((GRP == GRP_DENSE || GRP == GRP_SLOT) && FI::kAct16 && MB == 1 && !SL),
                "staged activations: dense or slot mode, 16-bit, one row block");
  // rows of the block (slot mode: the slot's token, operand row 0)
  [[maybe_unused]] const int blk_rows = GRP == GRP_SLOT ? 1 : min(16, M - m0);
  [[maybe_unused]] auto act_row = [&](int r) { return GRP == GRP_SLOT ? (int)blockIdx.z / p.topk : m0 + r; };
  extern __shared__ float red_dyn[];
  [[maybe_unused]] uint8_t* const a_lds =
      reinterpret_cast<uint8_t*>(red_dyn) + (size_t)W * (MB * NB * 4) * 64 * sizeof(float);
  // at or above 2^31: past every range (ranges stay below 2 GiB), and adding
  // the group offset cannot wrap
  constexpr int kOutOfRange = INT32_MIN;
  int aoff[MB];
  [[maybe_unused]] int aeoff[MB];  // E8M0 row offset of MXFP4 activations
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + 16 * mb + c;
    int row = -1;
    if constexpr (GRP == GRP_DENSE) {
      row = m < M ? m : -1;
    } else if constexpr (GRP == GRP_SLOT) {
      row = (mb == 0 && c == 0) ? (int)blockIdx.z / p.topk : -1;  // row 0: the slot's token
    } else if constexpr (GRP == GRP_TOKEN) {
      row = (mb == 0 && c == 0) ? 0 : -1;  // row 0; the step's slot row is a scalar offset
    } else {
      const int id = p.sorted_ids[m];
      if (id < p.n_slots) row = (GRP == GRP_GATHER) ? id / p.topk : m;
    }
    // 16-bit step t: bytes 256 g + 64 t + 16 kq; 8-bit piece h: 128 g + 64 h + 16 kq
    aoff[mb] = row >= 0 ? row * a_rowb + 16 * kq : kOutOfRange;
    aeoff[mb] = row >= 0 ? row * 4 : kOutOfRange;
  }
  int woff[NB], soff[NB], zoff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int f0 = nblk(nb) * GW;
    woff[nb] = f0 * kFragB + lane * ((FI::kW2 || FI::kW3) ? 8 : 16);
    soff[nb] = FI::kNV4   ? f0 * 128 + c * 8 + (kq >> 1) * 4
               : FI::kMX4 ? f0 * 64 + c * 4
                          : (mx_weights(FMT) ? f0 * 64 + (lane & ~3) : f0 * 32 + (c >> 1) * 4);
    zoff[nb] = f0 * 8 + (c >> 3) * 4;
  }

  auto load = [&](Stage<FMT, MB, NB>& st, int g) {
    // scalar (per-step) offsets: weight fragment, scales, zero points, activations
    int sw = g * kFragB, ss = g * 32, sz = g * 8, sa16 = g * 256, sa8 = g * 128;
    if constexpr (GRP == GRP_TOKEN) {
      const int j = g / p.ge, gin = g - j * p.ge;
      const int slot = (int)blockIdx.z * p.topk + j;
      const int e = p.topk_ids[slot];
      const bool ok = e >= 0 && e < p.num_experts;
      const int eu = ok ? e : 0;  // an out-of-range expert reads expert 0, weighted by zero
      sw = eu * (int)p.w_expert + gin * kFragB;
      ss = eu * (int)p.s_expert * 2 + gin * 32;
      sz = eu * (int)p.z_expert * 4 + gin * 8;
      sa16 = slot * a_rowb + gin * 256;
      sa8 = slot * a_rowb + gin * 128;
      st.gw = ok ? p.topk_w[slot] * (FI::kActScale ? p.a_scale[slot] : 1.f) : 0.f;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      if constexpr (FI::kW2 || FI::kW3) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rw, woff[nb], sw, 2);
        st.b[nb] = u4_t{(uint32_t)v[0], (uint32_t)v[1], 0u, 0u};
      } else {
        st.b[nb] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[nb], sw, 2));
      }
    if constexpr (FI::kW8) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        st.b2[nb] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[nb] + 1024, sw, 2));
    }
    if constexpr (FI::kW3) {
      // the 1-bit plane: bytes [512, 768) of the fragment, one word per lane
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        st.b2[nb] = u4_t{__builtin_amdgcn_raw_buffer_load_b32(rw, woff[nb] + 512 - 4 * lane, sw, 2), 0u, 0u, 0u};
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      // Step t of the 16-bit operand: k = 32 t + 8 kq + [0,8); piece h of the
      // 8-bit operand: k = 64 h + 16 kq + [0,16).  Per load instruction the
      // four lanes of one row read 64 contiguous bytes.
      if constexpr (FI::kAct16) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          st.a[mb][t] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[mb] + 64 * t, sa16, 0));
      } else if constexpr (FI::kAct4) {
        // block kq of the group: k = 32 kq + [0, 32), 16 bytes; its scale byte
        // is byte kq of the row's group word
        st.a[mb][0] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[mb], g * 64, 0));
        st.asc[mb] = __builtin_amdgcn_raw_buffer_load_b32(rae, aeoff[mb], g * a_rows * 4, 0);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          st.a[mb][h] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[mb] + 64 * h, sa8, 0));
      }
    }
    // Metadata comes in as whole dwords, decoded only at compute time, so
    // that no wait is needed until the stage's math.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (e8m0_meta(FMT)) {
        st.sraw[nb] = __builtin_amdgcn_raw_buffer_load_b32(re, soff[nb], g * byte_meta_frag(FMT), 0);
      } else {
        st.sraw[nb] = __builtin_amdgcn_raw_buffer_load_b32(rsc, soff[nb], ss, 0);
        st.zraw[nb] = __builtin_amdgcn_raw_buffer_load_b32(rz, zoff[nb], sz, 0);
      }
    }
  };
  // the lane's 16-bit scale / E8M0 byte out of its metadata dword
  auto sbits = [&](const Stage<FMT, MB, NB>& st, int nb) -> uint32_t {
    return mx_weights(FMT) ? (st.sraw[nb] >> (8 * (lane & 3))) & 0xFFu : (st.sraw[nb] >> (16 * (c & 1))) & 0xFFFFu;
  };
  auto zero_of = [&](const Stage<FMT, MB, NB>& st, int nb) -> uint32_t {
    return p.zp_fixed < 0 ? (st.zraw[nb] >> (4 * (c & 7))) & 0xFu : (uint32_t)p.zp_fixed;
  };

  f4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f4_t{0.f, 0.f, 0.f, 0.f};
  // the 16-bit operands' exponent pattern, held in a VGPR so that each
  // unpacked register is one v_and_or_b32 (mask literal, magic register)
  [[maybe_unused]] const uint32_t magic_v = opaque_vgpr(f16_act(FMT) ? 0x64006400u : 0x43004300u);
  // E8M0 block scales 2^0 and 2^9 for the scaled matrix instruction, held in
  // VGPRs: the instruction reads its scales from VGPRs only, and a uniform
  // constant left to the compiler may be placed in a scalar register.
  [[maybe_unused]] const int e8_one = (int)opaque_vgpr(127u);
  [[maybe_unused]] const int e8_nine = (int)opaque_vgpr(136u);

  // token mode: the step's top-k weight (and slot row scale) times the group scale
  auto gfac = [&](const Stage<FMT, MB, NB>& st) -> float {
    if constexpr (GRP == GRP_TOKEN) return st.gw;
    (void)st;
    return 1.f;
  };
  auto compute = [&](const Stage<FMT, MB, NB>& st, int g) {
    [[maybe_unused]] f4_t rs[MB];
    [[maybe_unused]] f4_t rs4[MB][4];  // MXINT4: the row sums of each MFMA step
    if constexpr (FI::kMX4) {
      const uint32_t one2 = f16_act(FMT) ? 0x3C003C00u : 0x3F803F80u;
      const u4_t ones = u4_t{one2, one2, one2, one2};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 4; ++t) rs4[mb][t] = mfma16<FMT>(st.a[mb][t], ones, f4_t{0.f, 0.f, 0.f, 0.f});
    } else if constexpr (FI::kAct16 && !FI::kNV4) {
      const uint32_t one2 = f16_act(FMT) ? 0x3C003C00u : 0x3F803F80u;
      const u4_t ones = u4_t{one2, one2, one2, one2};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        rs[mb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) rs[mb] = mfma16<FMT>(st.a[mb][t], ones, rs[mb]);
      }
    } else if constexpr (FMT == FMT_Q8) {
      const i8_t ones = i8_t{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                             0x38383838, 0x38383838, 0x38383838, 0x38383838};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        rs[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            cat8(st.a[mb][0], st.a[mb][1]), ones, f4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, e8_one, 0, e8_one);
    }

#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const u4_t w = st.b[nb];
      if constexpr (FI::kW8 || FI::kW3) {
        // INT8: q = 16 * high + low (two nibble planes); INT3: q = 4 * high
        // + low (a bit plane and a crumb plane).  P_h and P_l against the
        // exact offset operands (OFF + high), (OFF + low); the row sums
        // remove (H + 1) OFF + z, H = 16 or 4.
        constexpr float kH = FI::kW8 ? 16.f : 4.f;
        const uint32_t magic = magic_v;
        const float off = f16_act(FMT) ? 1024.f : 128.f;
        const u4_t w2 = st.b2[nb];
        f4_t Ph[MB], Pl[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) Ph[mb] = Pl[mb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u4_t bh = FI::kW8 ? w16_operand(w[t], magic) : w1_operand(w2[0], magic, t);
          const u4_t bl = FI::kW8 ? w16_operand(w2[t], magic) : w2_operand(w[t >> 1], magic, t & 1);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            Ph[mb] = mfma16<FMT>(st.a[mb][t], bh, Ph[mb]);
            Pl[mb] = mfma16<FMT>(st.a[mb][t], bl, Pl[mb]);
          }
        }
        const float s = gfac(st) * (p.scale_bf16 ? bf16_bits_to_float(sbits(st, nb)) : f16_bits_to_float(sbits(st, nb)));
        const float cz = (kH + 1.f) * off + (float)p.zp_fixed;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][nb][r] += s * (kH * Ph[mb][r] + Pl[mb][r] - cz * rs[mb][r]);
      } else if constexpr (FI::kNV4) {
        // weights dequantised exactly in registers (nvfp4_operand); no zero
        // point, so no row-sum correction
        const uint32_t sw = st.sraw[nb];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u4_t bop = nvfp4_operand<!f16_act(FMT)>(w[t], (sw >> (8 * t)) & 0xFFu);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma16<FMT>(st.a[mb][t], bop, acc[mb][nb]);
        }
      } else if constexpr (FI::kMX4) {
        // one E8M0 scale per MFMA step (32 k): per step P against the offset
        // codes OFF + (v + 8) and s_t (P - (OFF + 8) rowsum_t), s_t =
        // 2^(X_t - 127) times the element's implicit 2^-2
        const uint32_t magic = magic_v;
        const float cz = (f16_act(FMT) ? 1024.f : 128.f) + 8.f;
        const uint32_t xw = st.sraw[nb];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u4_t bop = w16_operand(w[t], magic);
          const uint32_t X = (xw >> (8 * t)) & 0xFFu;
          const float sc = X == 255u ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(1.0f, (int)X - 129);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const f4_t P = mfma16<FMT>(st.a[mb][t], bop, f4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mb][nb][r] += sc * (P[r] - cz * rs4[mb][t][r]);
          }
        }
      } else if constexpr (FI::kAct16) {
        const uint32_t magic = magic_v;
        const float off = f16_act(FMT) ? 1024.f : 128.f;
        f4_t P[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) P[mb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u4_t bop = FI::kW2 ? w2_operand(w[t >> 1], magic, t & 1) : w16_operand(w[t], magic);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) P[mb] = mfma16<FMT>(st.a[mb][t], bop, P[mb]);
        }
        const float s = gfac(st) * (p.scale_bf16 ? bf16_bits_to_float(sbits(st, nb)) : f16_bits_to_float(sbits(st, nb)));
        const float cz = off + (float)zero_of(st, nb);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][nb][r] += s * (P[mb][r] - cz * rs[mb][r]);
      } else if constexpr (FMT == FMT_I8) {
        const i4_t b0 = i4_t{(int)((w[0] << 4) & 0xF0F0F0F0u), (int)(w[0] & 0xF0F0F0F0u),
                             (int)((w[1] << 4) & 0xF0F0F0F0u), (int)(w[1] & 0xF0F0F0F0u)};
        const i4_t b1 = i4_t{(int)((w[2] << 4) & 0xF0F0F0F0u), (int)(w[2] & 0xF0F0F0F0u),
                             (int)((w[3] << 4) & 0xF0F0F0F0u), (int)(w[3] & 0xF0F0F0F0u)};
        const float s16 = gfac(st) * 0.0625f * (p.scale_bf16 ? bf16_bits_to_float(sbits(st, nb)) : f16_bits_to_float(sbits(st, nb)));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          i4_t P = i4_t{0, 0, 0, 0};
          P = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, st.a[mb][0]), b0, P, 0, 0, 0);
          P = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, st.a[mb][1]), b1, P, 0, 0, 0);
          if (p.i32_out) {
            const int n = (nt * NB + nb) * 16 + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int m = m0 + 16 * mb + 4 * kq + r;
              if (m < M) static_cast<int32_t*>(p.out)[((int64_t)m * N + n) * G + g] = P[r] >> 4;
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][nb][r] += s16 * (float)P[r];
        }
      } else if constexpr (FMT == FMT_Q8) {
        const i8_t bop = i8_t{(int)(w[0] & 0x0F0F0F0Fu), (int)((w[0] >> 4) & 0x0F0F0F0Fu),
                              (int)(w[1] & 0x0F0F0F0Fu), (int)((w[1] >> 4) & 0x0F0F0F0Fu),
                              (int)(w[2] & 0x0F0F0F0Fu), (int)((w[2] >> 4) & 0x0F0F0F0Fu),
                              (int)(w[3] & 0x0F0F0F0Fu), (int)((w[3] >> 4) & 0x0F0F0F0Fu)};
        const float s = gfac(st) * (p.scale_bf16 ? bf16_bits_to_float(sbits(st, nb)) : f16_bits_to_float(sbits(st, nb)));
        const float z = (float)zero_of(st, nb);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          // codes 0x00..0x0F are q * 2^-9 in e4m3; block scale 2^9 (E8M0 136) undoes it
          const f4_t P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              cat8(st.a[mb][0], st.a[mb][1]), bop, f4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, e8_one, 0, e8_nine);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][nb][r] += s * (P[r] - z * rs[mb][r]);
        }
      } else if constexpr (FMT == FMT_F44) {
        // fp4 x fp4: both operands E2M1 (format 4), each with its block scales
        const i8_t bop = i8_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
        const int sb = (int)sbits(st, nb);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u4_t x = st.a[mb][0];
          const i8_t av = i8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
          const int sa = (int)((st.asc[mb] >> (8 * kq)) & 0xFFu);
          acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bop, acc[mb][nb], 4, 4, 0, sa, 0, sb);
        }
      } else {  // FMT_F4
        const i8_t bop = i8_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
        const int sb = (int)sbits(st, nb);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              cat8(st.a[mb][0], st.a[mb][1]), bop, acc[mb][nb], 0, 4, 0, e8_one, 0, sb);
      }
    }
    (void)g;
  };

  // Software pipeline: STAGES groups of loads in flight ahead of the math.
  // Loads are issued without branches (a load past the end of this wave's
  // range re-reads group g_dummy, an in-range fragment that stays hot in L2)
  // so that the wait before each stage's math counts only that stage's loads.
  const int g_dummy = min(g_beg, G - 1);
  auto group_of = [&](int it) { return it < n_it ? my_first + it * W : g_dummy; };
  // The prologue issues the stages in order (no scheduling across the
  // barriers): the wait before stage d's math then counts the loads of the
  // later stages, on the first pass as in the loop.
  Stage<FMT, MB, NB> st[STAGES];
  if constexpr (AS) {
    // weights and metadata of group g (dense: no per-step expert)
    auto load_wm = [&](Stage<FMT, MB, NB>& s_, int g) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if constexpr (FI::kW2 || FI::kW3) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(rw, woff[nb], g * kFragB, 2);
          s_.b[nb] = u4_t{(uint32_t)v[0], (uint32_t)v[1], 0u, 0u};
        } else {
          s_.b[nb] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[nb], g * kFragB, 2));
        }
      if constexpr (FI::kW8) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          s_.b2[nb] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[nb] + 1024, g * kFragB, 2));
      }
      if constexpr (FI::kW3) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          s_.b2[nb] = u4_t{__builtin_amdgcn_raw_buffer_load_b32(rw, woff[nb] + 512 - 4 * lane, g * kFragB, 2), 0u, 0u, 0u};
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (e8m0_meta(FMT)) {
          s_.sraw[nb] = __builtin_amdgcn_raw_buffer_load_b32(re, soff[nb], g * byte_meta_frag(FMT), 0);
        } else {
          s_.sraw[nb] = __builtin_amdgcn_raw_buffer_load_b32(rsc, soff[nb], g * 32, 0);
          s_.zraw[nb] = __builtin_amdgcn_raw_buffer_load_b32(rz, zoff[nb], g * 8, 0);
        }
      }
    };
    constexpr int kWMLoads = NB * (1 + ((FI::kW8 || FI::kW3) ? 1 : 0) + (e8m0_meta(FMT) ? 1 : 2));
    // group g's operand of this lane's row, zero for rows past M
    auto load_a_lds = [&](Stage<FMT, MB, NB>& s_, int g) {
      const uint8_t* src = a_lds + c * p.a_pitch + (g - g_beg) * 256 + 16 * kq;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        s_.a[0][t] = c < blk_rows ? *reinterpret_cast<const u4_t*>(src + 64 * t) : u4_t{0u, 0u, 0u, 0u};
    };
    // The slab: blk_rows rows x ceil(span / 1 KiB) chunks, each one 64-lane
    // 16-byte load straight into LDS (a row's last chunk may run past this
    // split's groups into the row's padding; past the buffer it reads zeros).
    const int nch = ((g_end - g_beg) * 256 + 1023) >> 10;
    for (int idx = wave; idx < blk_rows * nch; idx += W) {
      const int r = idx / nch, ch = idx - r * nch;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(a_lds + r * p.a_pitch + ch * 1024), 16,
                                               act_row(r) * a_rowb + 16 * lane, g_beg * 256 + ch * 1024, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < STAGES; ++d) {
      load_wm(st[d], group_of(d));
      __builtin_amdgcn_sched_barrier(0);
    }
    // The slab copies went out first: with at most the prologue's weight and
    // metadata loads still in flight, this wave's copies have landed (loads
    // complete in order); the barrier then covers every wave's.
    static_assert(STAGES * kWMLoads < 64, "prologue loads exceed the counter");
    wait_vm<STAGES * kWMLoads>();
    __syncthreads();
#pragma unroll
    for (int d = 0; d < STAGES; ++d) load_a_lds(st[d], group_of(d));
    for (int i = 0; i < n_it; i += STAGES) {
#pragma unroll
      for (int d = 0; d < STAGES; ++d) {
        if (i + d < n_it) compute(st[d], my_first + (i + d) * W);
        const int gn = group_of(i + d + STAGES);
        load_wm(st[d], gn);
        load_a_lds(st[d], gn);
      }
    }
  } else {
#pragma unroll
    for (int d = 0; d < STAGES; ++d) {
      load(st[d], group_of(d));
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int i = 0; i < n_it; i += STAGES) {
#pragma unroll
      for (int d = 0; d < STAGES; ++d) {
        if (i + d < n_it) compute(st[d], my_first + (i + d) * W);
        load(st[d], group_of(i + d + STAGES));
      }
    }
  }

  if (p.i32_out) return;  // per-group accumulators already written

  // ---- reduce the W partial accumulators of this workgroup (fixed order) ----
  constexpr int E = MB * NB * 4;
  float* red;  // [W][E][64]
  if constexpr (SL) {
    __shared__ float red_st[(MAXT / 64) * E * 64];
    red = red_st;
  } else {
    red = red_dyn;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * E + (mb * NB + nb) * 4 + r) * 64 + lane] = acc[mb][nb][r];
  __syncthreads();

  const int S = gridDim.y;
  const int nthreads = blockDim.x;
  for (int e = threadIdx.x; e < E * 64; e += nthreads) {
    float v = 0.f;
    for (int w = 0; w < W; ++w) v += red[w * E * 64 + e];
    const int l = e & 63;
    const int idx = e >> 6;
    const int r = idx & 3;
    const int nb = (idx >> 2) % NB;
    const int mb = (idx >> 2) / NB;
    const int m = m0 + 16 * mb + 4 * (l >> 4) + r;
    const int n = nblk(nb) * 16 + (l & 15);
    if constexpr (GRP == GRP_TOKEN) {
      // row 0 is the token: the top-k weights are in, the sum over its slots is done
      if (m != m0) continue;
      store_out(p.out, (int64_t)blockIdx.z * N + n, v, p.out_bf16);
      continue;
    }
    if constexpr (GRP != GRP_DENSE) {
      // m is the row of the aligned slot array (slot mode: row 0 is the
      // block's slot); padding slots are dropped
      const int id = GRP == GRP_SLOT ? (m == m0 ? (int)blockIdx.z : p.n_slots) : p.sorted_ids[m];
      if (id >= p.n_slots) continue;
      const int tok = id / p.topk;
      const int64_t orow = GRP == GRP_SLOT ? id : m;  // output row: the slot (slot mode) or the aligned row
      if constexpr (GRP == GRP_GATHER || GRP == GRP_SLOT) {
        const float sa = FI::kActScale ? p.a_scale[tok] : 1.f;
        if (paired) {
          if (nb >= NB / 2) continue;
          float u = 0.f;  // the up projection of the same row and column
          for (int w = 0; w < W; ++w) u += red[w * E * 64 + e + (NB / 2) * 4 * 64];
          const float gv = v * sa;
          const float act = gv / (1.f + expf(-gv)) * (u * sa);  // SiLU(gate) * up
          const int half = N / 2;
          if (p.epi == GEPI_SILU) {
            store_out(p.out, orow * half + n, act, p.out_bf16);
          } else {
            p.f32_out[orow * half + n] = act;  // requantised to fp8 by moe_requant_kernel
          }
        } else {
          store_out(p.out, orow * N + n, v * sa, p.out_bf16);
        }
      } else {
        const float sa = FI::kActScale ? p.a_scale[m] : 1.f;
        p.rows16[(int64_t)id * N + n] = float_to_bf16_bits(v * sa * p.topk_w[id]);  // this slot's weighted row
      }
      continue;
    }
    if (m >= M) continue;
    if (FI::kActScale) v *= p.a_scale[m];
    if constexpr (FI::kNV4) v *= nv_scale;
    if (S == 1) {
      const uint16_t o = p.out_bf16 ? float_to_bf16_bits(v) : float_to_f16_bits(v);
      static_cast<uint16_t*>(p.out)[(int64_t)m * N + n] = o;
    } else {
      p.part[((int64_t)split * M + m) * N + n] = v;
    }
  }
#endif
}

}  // namespace hq
