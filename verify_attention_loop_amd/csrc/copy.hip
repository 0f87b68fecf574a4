// Writing planes into pages: the append path of the paged plane allocator.
// A page of plane p holds 16 consecutive positions of one (sequence, layer)
// for all KV heads: K token-major, V in four quads, quad g holding the tokens
// g, g + 4, g + 8, g + 12 interleaved per channel (layout in params.hpp).
#include <hip/hip_runtime.h>

#include "params.hpp"

namespace lkv {

template <int ES>
__global__ __launch_bounds__(256) void append_kernel(const CopyParams p, int D) {
  const int64_t total = (int64_t)p.n_tok * p.hkv * D;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const uint64_t head = (uint64_t)kPage * D * ES;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int c = (int)(idx % D);
    const int h = (int)((idx / D) % p.hkv);
    const int n = (int)(idx / ((int64_t)D * p.hkv));
    const int pos = p.pos0 + n;
    const int lp = pos / kPage - p.page0;
    const int s = pos % kPage;
    uint8_t* page = p.pool + (uint64_t)p.phys[lp] * p.page_bytes;
    uint8_t* kd = page + (uint64_t)h * head + ((uint64_t)s * D + c) * ES;
    uint8_t* vd = page + (uint64_t)p.hkv * head + (uint64_t)h * head +
                  ((uint64_t)(s % kQuad) * kQuad * D + (uint64_t)c * kQuad + (s / kQuad)) * ES;
    const uint8_t* ks = reinterpret_cast<const uint8_t*>(p.k) + idx * ES;
    const uint8_t* vs = reinterpret_cast<const uint8_t*>(p.v) + idx * ES;
    if constexpr (ES == 4) {
      *reinterpret_cast<uint32_t*>(kd) = *reinterpret_cast<const uint32_t*>(ks);
      *reinterpret_cast<uint32_t*>(vd) = *reinterpret_cast<const uint32_t*>(vs);
    } else {
      *reinterpret_cast<uint16_t*>(kd) = *reinterpret_cast<const uint16_t*>(ks);
      *reinterpret_cast<uint16_t*>(vd) = *reinterpret_cast<const uint16_t*>(vs);
    }
  }
}

__global__ __launch_bounds__(256) void fill_words_kernel(uint32_t* dst, int64_t n_words, uint32_t value) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride) dst[i] = value;
}

__global__ __launch_bounds__(256) void table_write_kernel(const TableWriteParams p) {
  for (int i = threadIdx.x; i < p.n; i += blockDim.x) p.dst[i] = p.vals[i];
}

static inline int grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  if (g > 16384) g = 16384;
  if (g < 1) g = 1;
  return (int)g;
}

hipError_t launch_append(const CopyParams& p, int dtype, int head_dim, hipStream_t s) {
  const int64_t total = (int64_t)p.n_tok * p.hkv * head_dim;
  if (total <= 0) return hipSuccess;
  if (dtype == 0) hipLaunchKernelGGL((append_kernel<4>), dim3(grid_for(total)), dim3(256), 0, s, p, head_dim);
  else hipLaunchKernelGGL((append_kernel<2>), dim3(grid_for(total)), dim3(256), 0, s, p, head_dim);
  return hipGetLastError();
}

// Fill n_bytes (a multiple of 4) at dst with a repeated 32-bit pattern.  A kernel
// rather than a memset so that it can sit inside a captured graph.
hipError_t launch_fill(void* dst, uint64_t n_bytes, uint32_t value, hipStream_t s) {
  const int64_t n = (int64_t)(n_bytes / 4);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_words_kernel, dim3(grid_for(n)), dim3(256), 0, s, reinterpret_cast<uint32_t*>(dst), n,
                     value);
  return hipGetLastError();
}

// Copy n block-table entries from host memory to dst (device) on the stream, in
// chunks carried as kernel arguments.
hipError_t launch_table_write(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s) {
  for (int64_t i0 = 0; i0 < n; i0 += kTableChunk) {
    TableWriteParams P;
    P.dst = dst + i0;
    P.n = (int32_t)(n - i0 < kTableChunk ? n - i0 : kTableChunk);
    for (int i = 0; i < P.n; ++i) P.vals[i] = src[i0 + i];
    hipLaunchKernelGGL(table_write_kernel, dim3(1), dim3(256), 0, s, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lkv
