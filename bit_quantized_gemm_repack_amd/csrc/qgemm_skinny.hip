// Launchers of the small-M ("skinny") kernel, qgemm_skinny_kernel.h: one
// instantiation per format x (row blocks, column blocks, stages, waves).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "launch.h"
#include "qgemm_skinny_kernel.h"

namespace hq {

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

template <typename Kern>
static hipError_t launch_kernel(Kern kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, const SkinnyArgs& a) {
  return launch_timed(kern, grid, block, lds, s, a);
}

// Instantiated shapes: up to 8 waves per workgroup (256 VGPRs per lane) for
// every (tile_m, tile_n, stages), and 16 waves (128 VGPRs per lane) for one
// column block of up to 16 rows.
template <int FMT, int MB, int NB>
static hipError_t launch_t(const SkinnyCfg& cfg, const SkinnyArgs& a, dim3 grid, dim3 block, size_t lds,
                           hipStream_t s) {
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
  const size_t lds = (size_t)cfg.waves * cfg.mb * cfg.nb * 4 * 64 * sizeof(float);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool slot = mode == GRP_SLOT;
  switch (fmt) {
    case FMT_W16F16:
      return (int)(slot ? launch_byslot_t<FMT_W16F16, GRP_SLOT>(cfg, a, grid, block, lds, s)
                        : launch_byslot_t<FMT_W16F16, GRP_TOKEN>(cfg, a, grid, block, lds, s));
    case FMT_W16BF16:
      return (int)(slot ? launch_byslot_t<FMT_W16BF16, GRP_SLOT>(cfg, a, grid, block, lds, s)
                        : launch_byslot_t<FMT_W16BF16, GRP_TOKEN>(cfg, a, grid, block, lds, s));
    case FMT_Q8:
      return (int)(slot ? launch_byslot_t<FMT_Q8, GRP_SLOT>(cfg, a, grid, block, lds, s)
                        : launch_byslot_t<FMT_Q8, GRP_TOKEN>(cfg, a, grid, block, lds, s));
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
  const size_t lds = (size_t)cfg.waves * cfg.mb * cfg.nb * 4 * 64 * sizeof(float);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (fmt) {
    case FMT_W16F16: return (int)launch_mb<FMT_W16F16>(cfg, a, grid, block, lds, s);
    case FMT_W16BF16: return (int)launch_mb<FMT_W16BF16>(cfg, a, grid, block, lds, s);
    case FMT_W8F16: return (int)launch_mb<FMT_W8F16>(cfg, a, grid, block, lds, s);
    case FMT_W8BF16: return (int)launch_mb<FMT_W8BF16>(cfg, a, grid, block, lds, s);
    case FMT_W2F16: return (int)launch_mb<FMT_W2F16>(cfg, a, grid, block, lds, s);
    case FMT_W2BF16: return (int)launch_mb<FMT_W2BF16>(cfg, a, grid, block, lds, s);
    case FMT_W3F16: return (int)launch_mb<FMT_W3F16>(cfg, a, grid, block, lds, s);
    case FMT_W3BF16: return (int)launch_mb<FMT_W3BF16>(cfg, a, grid, block, lds, s);
    case FMT_MX4F16: return (int)launch_mb<FMT_MX4F16>(cfg, a, grid, block, lds, s);
    case FMT_MX4BF16: return (int)launch_mb<FMT_MX4BF16>(cfg, a, grid, block, lds, s);
    case FMT_NV4F16: return (int)launch_mb<FMT_NV4F16>(cfg, a, grid, block, lds, s);
    case FMT_NV4BF16: return (int)launch_mb<FMT_NV4BF16>(cfg, a, grid, block, lds, s);
    case FMT_I8: return (int)launch_mb<FMT_I8>(cfg, a, grid, block, lds, s);
    case FMT_Q8: return (int)launch_mb<FMT_Q8>(cfg, a, grid, block, lds, s);
    case FMT_F4: return (int)launch_mb<FMT_F4>(cfg, a, grid, block, lds, s);
    case FMT_F44: return (int)launch_mb<FMT_F44>(cfg, a, grid, block, lds, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace hq
