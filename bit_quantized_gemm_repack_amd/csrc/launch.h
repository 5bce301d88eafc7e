// Kernel launch that honours the timing events armed for it (hq_time_next_launch):
// a launch with events goes through the extended launch, which records them
// at the dispatch's start and end on the device.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "hq_internal.h"

namespace hq {

template <typename Kern, typename... Args>
inline hipError_t launch_timed(Kern kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
  const TimingEvents ev = take_timing();
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, s, static_cast<hipEvent_t>(ev.start),
                          static_cast<hipEvent_t>(ev.stop), 0, args...);
  else
    hipLaunchKernelGGL(kern, grid, block, lds, s, args...);
  return hipGetLastError();
}

}  // namespace hq
