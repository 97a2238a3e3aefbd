// Launch of a kernel that a caller may time.  With timing events, the
// launch goes through hipExtLaunchKernelGGL, which records the two events
// at the kernel's own start and end; events recorded on the stream around
// an ordinary launch also hold the dispatch gap before the kernel starts,
// several microseconds against kernels of tens.  Without events it is an
// ordinary launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace pa_internal {

template <typename... Args, typename F = void (*)(Args...)>
inline void launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t stream, void *ev_begin,
                         void *ev_end, Args... args) {
  if (ev_begin || ev_end)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, reinterpret_cast<hipEvent_t>(ev_begin),
                          reinterpret_cast<hipEvent_t>(ev_end), 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
}

}  // namespace pa_internal
