// Streaming-read probe: the achievable HBM read rate on this GPU, the yardstick
// the attention kernels' bandwidth is compared with (next to the datasheet peak).
// It reads a buffer once with the same load form the page streams use (16-byte
// nontemporal loads, whole 1 KB runs per wave instruction, four loads in flight
// per lane) and writes nothing but a word that is never taken in practice (so
// the loads cannot be dropped).  No part of the attention path calls it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "launch.hpp"
#include "loopattn.h"

namespace lkv {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;
constexpr uint64_t kProbeChunk = (uint64_t)kProbeThreads * kProbeUnroll * 16;  // bytes per workgroup
static_assert(kProbeChunk == LKV_PROBE_CHUNK, "the probe's size unit is part of the C-ABI");

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint8_t* buf, uint32_t* sink) {
  const uint8_t* base = buf + (uint64_t)blockIdx.x * kProbeChunk + threadIdx.x * 16;
  u32x4_t v[kProbeUnroll];
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u)
    v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + u * (kProbeThreads * 16)));
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_probe_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s, const LaunchEvents& ev) {
  const uint64_t blocks = bytes / kProbeChunk;
  if (blocks == 0 || blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  const uint8_t* b = reinterpret_cast<const uint8_t*>(buf);
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(probe_read_kernel, dim3((uint32_t)blocks), dim3(kProbeThreads), 0, s, ev.start, ev.stop, 0u,
                          b, sink);
  else hipLaunchKernelGGL(probe_read_kernel, dim3((uint32_t)blocks), dim3(kProbeThreads), 0, s, b, sink);
  return hipGetLastError();
}

}  // namespace lkv
