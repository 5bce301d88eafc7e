// Launchers of the tiled kernel (qgemm_tiled_kernel.h) for every format but
// fp16 activations (qgemm_tiled_f16.hip).
#include "qgemm_tiled_kernel.h"

namespace hq {

int launch_tiled(int fmt, const TiledCfgRt& cfg, const TiledArgs& a, void* stream) {
  if (!splits_cover_k(cfg, a, true)) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n), (unsigned)(a.part ? cfg.split : 1));
  switch (fmt) {
    case FMT_W16F16:
    case FMT_W8F16:
    case FMT_W2F16:
    case FMT_W3F16: return (int)launch_tiled_f16(fmt, GRP_DENSE, cfg, a, grid, s);
    case FMT_W16BF16: return (int)launch_tiled_f<FMT_W16BF16, GRP_DENSE>(cfg, a, grid, s);
    case FMT_W8BF16: return (int)launch_tiled_f<FMT_W8BF16, GRP_DENSE>(cfg, a, grid, s);
    case FMT_W2BF16: return (int)launch_tiled_f<FMT_W2BF16, GRP_DENSE>(cfg, a, grid, s);
    case FMT_W3BF16: return (int)launch_tiled_f<FMT_W3BF16, GRP_DENSE>(cfg, a, grid, s);
    case FMT_MX4F16: return (int)launch_tiled_f<FMT_MX4F16, GRP_DENSE>(cfg, a, grid, s);
    case FMT_MX4BF16: return (int)launch_tiled_f<FMT_MX4BF16, GRP_DENSE>(cfg, a, grid, s);
    case FMT_NV4F16: return (int)launch_tiled_f16(fmt, GRP_DENSE, cfg, a, grid, s);
    case FMT_NV4BF16: return (int)launch_tiled_f<FMT_NV4BF16, GRP_DENSE>(cfg, a, grid, s);
    case FMT_I8: return (int)launch_tiled_f<FMT_I8, GRP_DENSE>(cfg, a, grid, s);
    case FMT_Q8: return (int)launch_tiled_f<FMT_Q8, GRP_DENSE>(cfg, a, grid, s);
    case FMT_F4: return (int)launch_tiled_f<FMT_F4, GRP_DENSE>(cfg, a, grid, s);
    case FMT_F44: return (int)launch_tiled_f<FMT_F44, GRP_DENSE>(cfg, a, grid, s);
  }
  return (int)hipErrorInvalidValue;
}

int launch_tiled_grouped(int fmt, int mode, const TiledCfgRt& cfg, const TiledArgs& a, int64_t blocks,
                         void* stream) {
  if (!splits_cover_k(cfg, a, false) || a.part) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool paired = mode == GRP_GATHER && (a.epi == GEPI_SILU || a.epi == GEPI_SILU_F32);
  const int bn = 64 * cfg.nbw;
  const int ntiles = paired ? (a.N / 2) / (bn / 2) : a.N / bn;
  const dim3 grid((unsigned)ntiles, (unsigned)blocks);
  if (mode == GRP_GATHER) {
    switch (fmt) {
      case FMT_W16F16: return (int)launch_tiled_f16(fmt, GRP_GATHER, cfg, a, grid, s);
      case FMT_W16BF16: return (int)launch_tiled_f<FMT_W16BF16, GRP_GATHER>(cfg, a, grid, s);
      case FMT_Q8: return (int)launch_tiled_f<FMT_Q8, GRP_GATHER>(cfg, a, grid, s);
    }
  } else if (mode == GRP_SORTED) {
    switch (fmt) {
      case FMT_W16F16: return (int)launch_tiled_f16(fmt, GRP_SORTED, cfg, a, grid, s);
      case FMT_W16BF16: return (int)launch_tiled_f<FMT_W16BF16, GRP_SORTED>(cfg, a, grid, s);
      case FMT_Q8: return (int)launch_tiled_f<FMT_Q8, GRP_SORTED>(cfg, a, grid, s);
    }
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace hq
