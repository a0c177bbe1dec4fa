// hq_launch.hpp — the kernel launch helper of the kernel files (HIP sources only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "hq_internal.hpp"

namespace hq {

// Launch a kernel; with a recording token its events take the kernel's start and end times.
template <class K, class... A>
inline hipError_t launch_k(K kernel, dim3 grid, dim3 block, hipStream_t st, int tok, A... args) {
  hipEvent_t e0, e1;
  prof_events(tok, &e0, &e1);
  if (e0) hipExtLaunchKernelGGL(kernel, grid, block, 0, st, e0, e1, 0, args...);
  else hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  return hipGetLastError();
}

}  // namespace hq
