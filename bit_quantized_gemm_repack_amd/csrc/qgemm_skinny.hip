// Launchers of the small-M ("skinny") kernel, qgemm_skinny_kernel.h: one
// instantiation per format x (row blocks, column blocks, stages, waves).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>
#include <utility>
#include <vector>

#include "launch.h"
#include "qgemm_skinny_kernel.h"

namespace hq {

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

// LDS per workgroup the staged activation slab may bring the dense launch to
// (the CU's whole LDS).
constexpr int64_t kSkinnyMaxLds = 160 * 1024;

// A launch with more than the default 64 KiB of dynamic LDS needs the
// kernel's limit raised, once per kernel and device.
static hipError_t allow_lds(const void* kern, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::vector<std::pair<int, const void*>> done;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : done)
    if (d.first == dev && d.second == kern) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkinnyMaxLds);
  if (e == hipSuccess) done.emplace_back(dev, kern);
  return e;
}

template <typename Kern>
static hipError_t launch_kernel(Kern kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, const SkinnyArgs& a) {
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern), lds);
  if (e != hipSuccess) return e;
  return launch_timed(kern, grid, block, lds, s, a);
}

// CUs of the current device (the launch heuristics' count of workgroups per CU).
static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return cus > 0 ? cus : 256;
}

// Vector-memory loads of weights and metadata per group and wave.
constexpr int wm_loads(int fmt, int nb) {
  return nb * (1 + ((w8_weights(fmt) || w3_weights(fmt)) ? 1 : 0) + (e8m0_meta(fmt) ? 1 : 2));
}

// Whether the staged-activation variant (AS = 1) exists for this shape: 16-bit
// activations, one row block, 2 or 4 stages whose prologue loads the wait
// counter can hold.
constexpr bool stageable(int fmt, int mb, int nb, int stages) {
  return act16_fmt(fmt) && mb == 1 && (stages == 2 || stages == 4) && stages * wm_loads(fmt, nb) < 64;
}

template <int FMT, int NB, int ST, int MAXT>
static hipError_t launch_staged(const SkinnyArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  if constexpr (stageable(FMT, 1, NB, ST))
    return launch_kernel(qgemm_skinny<FMT, 1, NB, ST, MAXT, GRP_DENSE, 0, 0, 0, 0, 1>, grid, block, lds, s, a);
  return hipErrorInvalidValue;
}

// Instantiated shapes: up to 8 waves per workgroup (256 VGPRs per lane) for
// every (tile_m, tile_n, stages), and 16 waves (128 VGPRs per lane) for one
// column block of up to 16 rows; the staged-activation variants of the
// one-row-block shapes with 2 or 4 stages.
template <int FMT, int MB, int NB>
static hipError_t launch_t(const SkinnyCfg& cfg, const SkinnyArgs& a, dim3 grid, dim3 block, size_t lds,
                           hipStream_t s) {
  if constexpr (MB == 1 && act16_fmt(FMT)) {
    if (a.a_pitch > 0) {
      const bool two = cfg.stages <= 2;
      if (cfg.waves > 8) {
        if constexpr (NB == 1)
          return two ? launch_staged<FMT, 1, 2, 1024>(a, grid, block, lds, s)
                     : launch_staged<FMT, 1, 4, 1024>(a, grid, block, lds, s);
        return hipErrorInvalidValue;
      }
      return two ? launch_staged<FMT, NB, 2, 512>(a, grid, block, lds, s)
                 : launch_staged<FMT, NB, 4, 512>(a, grid, block, lds, s);
    }
  }
  if (cfg.waves > 8) {
    if constexpr (MB == 1 && NB == 1) {
      if (cfg.stages <= 2) return launch_kernel(qgemm_skinny<FMT, 1, 1, 2, 1024, GRP_DENSE>, grid, block, lds, s, a);
      return launch_kernel(qgemm_skinny<FMT, 1, 1, 4, 1024, GRP_DENSE>, grid, block, lds, s, a);
    }
    return hipErrorInvalidValue;
  }
  if (cfg.stages <= 2) return launch_kernel(qgemm_skinny<FMT, MB, NB, 2, 512, GRP_DENSE>, grid, block, lds, s, a);
  if (cfg.stages <= 4) return launch_kernel(qgemm_skinny<FMT, MB, NB, 4, 512, GRP_DENSE>, grid, block, lds, s, a);
  if constexpr (MB == 1 && NB <= 2)
    return launch_kernel(qgemm_skinny<FMT, MB, NB, 8, 512, GRP_DENSE>, grid, block, lds, s, a);
  return hipErrorInvalidValue;
}

template <int FMT, int MB>
static hipError_t launch_nb(const SkinnyCfg& cfg, const SkinnyArgs& a, dim3 grid, dim3 block, size_t lds,
                            hipStream_t s) {
  switch (cfg.nb) {
    case 1: return launch_t<FMT, MB, 1>(cfg, a, grid, block, lds, s);
    case 2: return launch_t<FMT, MB, 2>(cfg, a, grid, block, lds, s);
    case 4: return launch_t<FMT, MB, 4>(cfg, a, grid, block, lds, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT>
static hipError_t launch_mb(const SkinnyCfg& cfg, const SkinnyArgs& a, dim3 grid, dim3 block, size_t lds,
                            hipStream_t s) {
  switch (cfg.mb) {
    case 1: return launch_nb<FMT, 1>(cfg, a, grid, block, lds, s);
    case 2: return launch_nb<FMT, 2>(cfg, a, grid, block, lds, s);
    case 4: return launch_nb<FMT, 4>(cfg, a, grid, block, lds, s);
  }
  return hipErrorInvalidValue;
}

// Grouped instantiations: 16-row expert blocks, 2 (gate_up pair) or 4
// column blocks, two groups of loads in flight, up to 8 waves.
template <int FMT, int GRP>
static hipError_t launch_grouped_t(const SkinnyCfg& cfg, const SkinnyArgs& a, dim3 grid, dim3 block, size_t lds,
                                   hipStream_t s) {
  if (cfg.stages != 2 || cfg.waves > 8) return hipErrorInvalidValue;
  if (cfg.mb == 1 && cfg.nb == 2) return launch_kernel(qgemm_skinny<FMT, 1, 2, 2, 512, GRP>, grid, block, lds, s, a);
  if (cfg.mb == 1 && cfg.nb == 4) return launch_kernel(qgemm_skinny<FMT, 1, 4, 2, 512, GRP>, grid, block, lds, s, a);
  if (cfg.mb == 2 && cfg.nb == 2) return launch_kernel(qgemm_skinny<FMT, 2, 2, 2, 512, GRP>, grid, block, lds, s, a);
  if (cfg.mb == 2 && cfg.nb == 4) return launch_kernel(qgemm_skinny<FMT, 2, 4, 2, 512, GRP>, grid, block, lds, s, a);
  return hipErrorInvalidValue;
}

template <int FMT>
static hipError_t launch_grouped_f(int mode, const SkinnyCfg& cfg, const SkinnyArgs& a, dim3 grid, dim3 block,
                                   size_t lds, hipStream_t s) {
  if (mode == GRP_GATHER) return launch_grouped_t<FMT, GRP_GATHER>(cfg, a, grid, block, lds, s);
  if (mode == GRP_SORTED) return launch_grouped_t<FMT, GRP_SORTED>(cfg, a, grid, block, lds, s);
  return hipErrorInvalidValue;
}

int launch_skinny_grouped(int fmt, int mode, const SkinnyCfg& cfg, const SkinnyArgs& a, int64_t blocks,
                          void* stream) {
  if (a.G < 1 || a.gps != a.G || cfg.split != 1) return (int)hipErrorInvalidValue;
  const bool paired = mode == GRP_GATHER && (a.epi == GEPI_SILU || a.epi == GEPI_SILU_F32);
  const int ntiles = paired ? (a.N / 2) / (16 * (cfg.nb / 2)) : a.N / (16 * cfg.nb);
  dim3 grid(ntiles, 1, (unsigned)blocks);
  dim3 block(64 * cfg.waves);
  const size_t lds = (size_t)cfg.waves * cfg.mb * cfg.nb * 4 * 64 * sizeof(float);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (fmt) {
    case FMT_W16F16: return (int)launch_grouped_f<FMT_W16F16>(mode, cfg, a, grid, block, lds, s);
    case FMT_W16BF16: return (int)launch_grouped_f<FMT_W16BF16>(mode, cfg, a, grid, block, lds, s);
    case FMT_Q8: return (int)launch_grouped_f<FMT_Q8>(mode, cfg, a, grid, block, lds, s);
  }
  return (int)hipErrorInvalidValue;
}

// Slot and token modes (no alignment): one row per block, up to 16 waves.
template <int FMT, int GRP>
static hipError_t launch_byslot_t(const SkinnyCfg& cfg, const SkinnyArgs& a, dim3 grid, dim3 block, size_t lds,
                                  hipStream_t s) {
  if (cfg.stages != 2 || cfg.mb != 1 || cfg.waves > 16) return hipErrorInvalidValue;
  if constexpr (GRP == GRP_SLOT && act16_fmt(FMT)) {
    if (a.a_pitch > 0) {  // the slot's token row staged in LDS
      if (cfg.nb == 2) return launch_kernel(qgemm_skinny<FMT, 1, 2, 2, 1024, GRP, 0, 0, 0, 0, 1>, grid, block, lds, s, a);
      return hipErrorInvalidValue;
    }
  }
  if constexpr (GRP == GRP_TOKEN)
    if (cfg.nb == 1) return launch_kernel(qgemm_skinny<FMT, 1, 1, 2, 1024, GRP>, grid, block, lds, s, a);
  if (cfg.nb == 2) return launch_kernel(qgemm_skinny<FMT, 1, 2, 2, 1024, GRP>, grid, block, lds, s, a);
  if (cfg.nb == 4) return launch_kernel(qgemm_skinny<FMT, 1, 4, 2, 1024, GRP>, grid, block, lds, s, a);
  return hipErrorInvalidValue;
}

int launch_skinny_byslot(int fmt, int mode, const SkinnyCfg& cfg, const SkinnyArgs& a, int64_t blocks,
                         void* stream) {
  if (a.G < 1 || a.gps != a.G || cfg.split != 1 || blocks < 1 || blocks > 65535) return (int)hipErrorInvalidValue;
  if (mode != GRP_SLOT && mode != GRP_TOKEN) return (int)hipErrorInvalidValue;
  const bool paired = mode == GRP_SLOT && (a.epi == GEPI_SILU || a.epi == GEPI_SILU_F32);
  if (paired && cfg.nb < 2) return (int)hipErrorInvalidValue;
  const int ntiles = paired ? (a.N / 2) / (16 * (cfg.nb / 2)) : a.N / (16 * cfg.nb);
  dim3 grid(ntiles, 1, (unsigned)blocks);
  dim3 block(64 * cfg.waves);
  size_t lds = (size_t)cfg.waves * cfg.mb * cfg.nb * 4 * 64 * sizeof(float);
  const bool slot = mode == GRP_SLOT;
  // slot mode, 16-bit activations, two column blocks (the gate and up block
  // pair; with four, the staged form of the 1024-thread kernel spills): the
  // slot's token row over all of K staged in LDS behind the reduction buffer
  // (as the dense calls of a few rows), while it leaves room for the
  // workgroups each CU has to hold
  SkinnyArgs b = a;
  b.a_pitch = 0;
  if (slot && act16_fmt(fmt) && cfg.nb == 2) {
    const int64_t pitch = ((int64_t)a.G * 256 + 1023) / 1024 * 1024 + 16;
    static const int cus = device_cus();
    const int64_t per_cu = ((int64_t)ntiles * blocks + cus - 1) / cus;
    if (((int64_t)lds + pitch) * per_cu <= kSkinnyMaxLds) {
      b.a_pitch = (int)pitch;
      lds += (size_t)pitch;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (fmt) {
    case FMT_W16F16:
      return (int)(slot ? launch_byslot_t<FMT_W16F16, GRP_SLOT>(cfg, b, grid, block, lds, s)
                        : launch_byslot_t<FMT_W16F16, GRP_TOKEN>(cfg, b, grid, block, lds, s));
    case FMT_W16BF16:
      return (int)(slot ? launch_byslot_t<FMT_W16BF16, GRP_SLOT>(cfg, b, grid, block, lds, s)
                        : launch_byslot_t<FMT_W16BF16, GRP_TOKEN>(cfg, b, grid, block, lds, s));
    case FMT_Q8:
      return (int)(slot ? launch_byslot_t<FMT_Q8, GRP_SLOT>(cfg, b, grid, block, lds, s)
                        : launch_byslot_t<FMT_Q8, GRP_TOKEN>(cfg, b, grid, block, lds, s));
  }
  return (int)hipErrorInvalidValue;
}

int launch_skinny(int fmt, const SkinnyCfg& cfg, const SkinnyArgs& a, void* stream) {
  // every split holds at least one group, and the splits cover K
  if (a.G < 1 || a.gps < 1 || (int64_t)(cfg.split - 1) * a.gps >= a.G || (int64_t)cfg.split * a.gps < a.G)
    return (int)hipErrorInvalidValue;
  const int ntiles = a.N / (16 * cfg.nb);
  const int mchunks = (a.M + 16 * cfg.mb - 1) / (16 * cfg.mb);
  dim3 grid(ntiles, cfg.split, mchunks);
  dim3 block(64 * cfg.waves);
  size_t lds = (size_t)cfg.waves * cfg.mb * cfg.nb * 4 * 64 * sizeof(float);
  // Stage the activations in LDS (16-bit activations, up to 4 rows) while the
  // slab, behind the reduction buffer, leaves room for the workgroups each CU
  // has to hold: rows of the split's groups padded to whole KiB (the copy's
  // unit) plus 16 bytes, so that the rows start on different LDS banks.  On
  // the decode shapes on MI355X this took 0.1-1.1 us off every call of 1 and
  // 4 rows and added 0.1-1.3 us to those of 16 and 64 rows (a 16-row slab is
  // four times the bytes to copy before the first group's math).
  SkinnyArgs b = a;
  b.a_pitch = 0;
  const int st_eff = cfg.stages <= 2 ? 2 : (cfg.stages <= 4 ? 4 : cfg.stages);
  if (a.M <= 4 && stageable(fmt, cfg.mb, cfg.nb, st_eff) && (cfg.waves <= 8 || cfg.nb == 1) && !a.i32_out) {
    const int64_t pitch = ((int64_t)a.gps * 256 + 1023) / 1024 * 1024 + 16;
    const int64_t rows = a.M;
    const int64_t total = (int64_t)lds + rows * pitch;
    static const int cus = device_cus();
    const int64_t blocks = (int64_t)ntiles * cfg.split * mchunks;
    const int64_t per_cu = (blocks + cus - 1) / cus;
    if (total * per_cu <= kSkinnyMaxLds) {
      b.a_pitch = (int)pitch;
      lds = (size_t)total;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (fmt) {
    case FMT_W16F16: return (int)launch_mb<FMT_W16F16>(cfg, b, grid, block, lds, s);
    case FMT_W16BF16: return (int)launch_mb<FMT_W16BF16>(cfg, b, grid, block, lds, s);
    case FMT_W8F16: return (int)launch_mb<FMT_W8F16>(cfg, b, grid, block, lds, s);
    case FMT_W8BF16: return (int)launch_mb<FMT_W8BF16>(cfg, b, grid, block, lds, s);
    case FMT_W2F16: return (int)launch_mb<FMT_W2F16>(cfg, b, grid, block, lds, s);
    case FMT_W2BF16: return (int)launch_mb<FMT_W2BF16>(cfg, b, grid, block, lds, s);
    case FMT_W3F16: return (int)launch_mb<FMT_W3F16>(cfg, b, grid, block, lds, s);
    case FMT_W3BF16: return (int)launch_mb<FMT_W3BF16>(cfg, b, grid, block, lds, s);
    case FMT_MX4F16: return (int)launch_mb<FMT_MX4F16>(cfg, b, grid, block, lds, s);
    case FMT_MX4BF16: return (int)launch_mb<FMT_MX4BF16>(cfg, b, grid, block, lds, s);
    case FMT_NV4F16: return (int)launch_mb<FMT_NV4F16>(cfg, b, grid, block, lds, s);
    case FMT_NV4BF16: return (int)launch_mb<FMT_NV4BF16>(cfg, b, grid, block, lds, s);
    case FMT_I8: return (int)launch_mb<FMT_I8>(cfg, b, grid, block, lds, s);
    case FMT_Q8: return (int)launch_mb<FMT_Q8>(cfg, b, grid, block, lds, s);
    case FMT_F4: return (int)launch_mb<FMT_F4>(cfg, b, grid, block, lds, s);
    case FMT_F44: return (int)launch_mb<FMT_F44>(cfg, b, grid, block, lds, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace hq
