// Kernel launch helper with the library's opt-in per-kernel timing.
//
// While timing is enabled (moe_profile_begin), launches go through hipExtLaunchKernel
// with a start/stop event pair, so the elapsed time is the dispatch's own execution
// window on the stream it runs on; otherwise a plain launch.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace moe {

enum KernelKind : int {
  K_ROUTE = 0, K_GATEUP = 1, K_DOWN = 2, K_QUANT = 3, K_FILL = 4, K_TOPK = 5, K_HQUANT = 6,
  K_COMBINE = 7, K_KINDS = 8
};

bool profiling_enabled();
// A start/stop event pair registered under `kind`; false if none could be created.
bool profile_events(int kind, hipEvent_t* start, hipEvent_t* stop);

template <class K, class... A>
hipError_t launch_kernel(int kind, K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         A... args) {
  hipEvent_t e0, e1;
  if (profiling_enabled() && profile_events(kind, &e0, &e1)) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, e0, e1, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
  return hipGetLastError();
}

}  // namespace moe
