// Attention kernel launches with optional timing events.
//
// When a caller passes events, the kernel is launched with hipExtLaunchKernelGGL,
// which stamps the events with the start and the end of that kernel's own
// dispatch: no separate marker packets on the stream, so timing one launch does
// not add to the time it measures.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace lkv {

struct LaunchEvents {
  hipEvent_t start = nullptr;  // stamped when the launch starts (or null)
  hipEvent_t stop = nullptr;   // stamped when it ends (or null)
};

template <typename K, typename P>
inline void launch_k(K kernel, dim3 grid, dim3 block, hipStream_t s, const LaunchEvents& ev, const P& p) {
  if (ev.start || ev.stop) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0u, p);
  else hipLaunchKernelGGL(kernel, grid, block, 0, s, p);
}

}  // namespace lkv
