// Kernel launch with the optional timing events of akv_time_next_call.
//
// The events travel with the kernel dispatch (hipExtLaunchKernel): the start event
// takes the time the first kernel of an entry point starts, the stop event the time
// its last kernel ends, without the marker packets of hipEventRecord in between.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "internal.h"

namespace akv {

template <typename F, typename... Args>
inline void launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t s, bool first, bool last, Args... args) {
  const LaunchEvents& ev = active_events();
  hipExtLaunchKernelGGL(kernel, grid, block, 0, s, first ? (hipEvent_t)ev.start : nullptr,
                        last ? (hipEvent_t)ev.stop : nullptr, 0, args...);
}

}  // namespace akv
