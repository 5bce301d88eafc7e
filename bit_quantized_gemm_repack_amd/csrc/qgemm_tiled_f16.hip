// Launchers of the tiled kernel (qgemm_tiled_kernel.h) for fp16 activations,
// in a translation unit of their own: built with the matrix-instruction
// results in accumulation registers (the fp16 k loop has no per-group
// epilogue, so the accumulators stay there until the end).
#include "qgemm_tiled_kernel.h"

namespace hq {

hipError_t launch_tiled_f16(int fmt, int mode, const TiledCfgRt& cfg, const TiledArgs& a, dim3 grid, hipStream_t s) {
  if (fmt == FMT_W8F16) return mode == GRP_DENSE ? launch_tiled_f<FMT_W8F16, GRP_DENSE>(cfg, a, grid, s) : hipErrorInvalidValue;
  if (fmt == FMT_W2F16) return mode == GRP_DENSE ? launch_tiled_f<FMT_W2F16, GRP_DENSE>(cfg, a, grid, s) : hipErrorInvalidValue;
  if (fmt == FMT_NV4F16) return mode == GRP_DENSE ? launch_tiled_f<FMT_NV4F16, GRP_DENSE>(cfg, a, grid, s) : hipErrorInvalidValue;
  if (fmt == FMT_W3F16) return mode == GRP_DENSE ? launch_tiled_f<FMT_W3F16, GRP_DENSE>(cfg, a, grid, s) : hipErrorInvalidValue;
  switch (mode) {
    case GRP_DENSE: return launch_tiled_f<FMT_W16F16, GRP_DENSE>(cfg, a, grid, s);
    case GRP_GATHER: return launch_tiled_f<FMT_W16F16, GRP_GATHER>(cfg, a, grid, s);
    case GRP_SORTED: return launch_tiled_f<FMT_W16F16, GRP_SORTED>(cfg, a, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hq
