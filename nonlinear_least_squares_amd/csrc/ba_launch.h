// Kernel launch through the dispatch packet, so that a pair of timing events
// set by the profiler (dispatch_events) is recorded by the kernel's own
// dispatch and times the kernel alone.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "ba_kernels.h"

namespace ba {

template <typename... KArgs, typename... Args>
inline void launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                         uint32_t shmem, Args... args) {
  DispatchEvents& ev = dispatch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0u,
                        static_cast<KArgs>(args)...);
  if (ev.start) {
    ev.used = true;
    ev.start = ev.stop = nullptr;
  }
}

}  // namespace ba
