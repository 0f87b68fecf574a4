// GPU fill kernels for the seeded synthetic inputs (see synth.h).
// Input generation only; no attention arithmetic lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth.h"

using namespace synth;

namespace {

constexpr int kMaxQSeqs = 64;

struct QRows {
  int32_t seq[kMaxQSeqs];
  int32_t t0[kMaxQSeqs];
};

// Coefficient 0.88^k by k repeated fp64 multiplications, then rounded to fp32.
__device__ inline float ripen_coef(int k) {
  double c = 1.0;
  for (int i = 0; i < k; ++i) c *= 0.88;
  return (float)c;
}

__global__ void fill_kv_kernel(void* dst, int dtype, uint64_t seed, uint32_t tensor, uint32_t seq,
                               uint32_t layer, uint32_t plane, int n_heads, int d, int pos0,
                               int n_pos, int mode, int n_loops, float scale) {
  const int64_t total = (int64_t)n_pos * n_heads * d;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const uint32_t deepest = (uint32_t)(n_loops - 1);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int c = (int)(idx % d);
    const int h = (int)((idx / d) % n_heads);
    const int p = (int)(idx / ((int64_t)d * n_heads));
    const uint64_t elem = (uint64_t)(pos0 + p) * (uint64_t)d + (uint64_t)c;
    // mode 1: noise 0.88^(R-1-r) (the workload's recipe); mode 2: 0.88^(r+1) (the page's direction)
    const bool ripen = (mode == 1 || mode == 2) && (plane != deepest);
    const int coef_k = mode == 1 ? (int)(deepest - plane) : (int)plane + 1;
    const uint32_t base_plane = ripen ? deepest : plane;
    const float base = normal_f32(stream_key(seed, tensor, seq, layer, base_plane, h), elem) * scale;
    if (dtype == 0) {
      float out = base;
      if (ripen) {
        const float noise = normal_f32(stream_key(seed, tensor + 3u, seq, layer, plane, h), elem) * scale;
        const float coef = ripen_coef(coef_k);
        out = (float)__dadd_rn((double)base, __dmul_rn((double)coef, (double)noise));
      }
      ((float*)dst)[idx] = out;
    } else {
      uint16_t out = bf16_from_f32(base);
      if (ripen) {
        const float noise = normal_f32(stream_key(seed, tensor + 3u, seq, layer, plane, h), elem) * scale;
        const float coef = ripen_coef(coef_k);
        const double sum = __dadd_rn((double)f32_from_bf16(out), __dmul_rn((double)coef, (double)noise));
        out = bf16_from_f64(sum);
      }
      ((uint16_t*)dst)[idx] = out;
    }
  }
}

__global__ void fill_q_kernel(void* dst, int dtype, uint64_t seed, QRows rows, uint32_t layer,
                              uint32_t loop, int n_seqs, int q_len, int n_heads, int d, float scale) {
  const int64_t total = (int64_t)n_seqs * q_len * n_heads * d;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int c = (int)(idx % d);
    const int h = (int)((idx / d) % n_heads);
    const int i = (int)((idx / ((int64_t)d * n_heads)) % q_len);
    const int b = (int)(idx / ((int64_t)d * n_heads * q_len));
    const uint64_t elem = (uint64_t)(rows.t0[b] + i) * (uint64_t)d + (uint64_t)c;
    const float x = normal_f32(stream_key(seed, kQ, (uint32_t)rows.seq[b], layer, loop, h), elem) * scale;
    if (dtype == 0) ((float*)dst)[idx] = x;
    else ((uint16_t*)dst)[idx] = bf16_from_f32(x);
  }
}

__global__ void fill_codes_kernel(uint8_t* dst, uint64_t seed, uint32_t tensor, uint32_t seq,
                                  uint32_t layer, uint32_t plane, int n_heads, int d, int pos0,
                                  int n_pos, int bits) {
  const int64_t total = (int64_t)n_pos * n_heads * d;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int c = (int)(idx % d);
    const int h = (int)((idx / d) % n_heads);
    const int p = (int)(idx / ((int64_t)d * n_heads));
    const uint64_t elem = (uint64_t)(pos0 + p) * (uint64_t)d + (uint64_t)c;
    dst[idx] = (uint8_t)binom_code(stream_key(seed, tensor, seq, layer, plane, h), elem, bits);
  }
}

__global__ void fill_meta_kernel(uint16_t* dst, uint64_t seed, uint32_t t_scale, uint32_t t_zero,
                                 uint32_t seq, uint32_t layer, uint32_t plane, int n_heads, int n_ch,
                                 int row0, int n_rows, int bits) {
  const int64_t total = (int64_t)n_rows * n_heads * n_ch;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const float base = bits == 4 ? 0.5f : 1.0f;
  const float mid = bits == 4 ? 7.5f : 1.5f;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int c = (int)(idx % n_ch);
    const int h = (int)((idx / n_ch) % n_heads);
    const int r = (int)(idx / ((int64_t)n_ch * n_heads));
    const uint64_t elem = (uint64_t)(row0 + r) * (uint64_t)n_ch + (uint64_t)c;
    const uint32_t u = (uint32_t)(draw(stream_key(seed, t_scale, seq, layer, plane, h), elem) & kMask20);
    const float sigma32 = base * (1.0f + (float)u * (1.0f / 2097152.0f));
    const uint16_t s16 = f16_from_f32(sigma32);
    // fp16 -> fp32 is exact; do it with integer ops to stay independent of half intrinsics.
    const uint32_t sh = s16;
    const uint32_t e = (sh >> 10) & 0x1Fu, m = sh & 0x3FFu;
    const float s_back = bits_f32(((e + 112u) << 23) | (m << 13));  // sigma is a normal fp16
    const float n = normal_f32(stream_key(seed, t_zero, seq, layer, plane, h), elem);
    const float z32 = __fadd_rn(__fmul_rn(-mid, s_back), 0.125f * n);
    dst[2 * idx] = s16;
    dst[2 * idx + 1] = f16_from_f32(z32);
  }
}

inline int grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

int synth_fill_kv(void* dst, int dtype, uint64_t seed, int tensor, int seq, int layer, int plane,
                  int n_heads, int d, int pos0, int n_pos, int mode, int n_loops, float scale,
                  void* stream) {
  const int64_t total = (int64_t)n_pos * n_heads * d;
  if (total <= 0) return 0;
  hipLaunchKernelGGL(fill_kv_kernel, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)stream, dst,
                     dtype, seed, (uint32_t)tensor, (uint32_t)seq, (uint32_t)layer, (uint32_t)plane,
                     n_heads, d, pos0, n_pos, mode, n_loops, scale);
  return (int)hipGetLastError();
}

int synth_fill_q(void* dst, int dtype, uint64_t seed, const int32_t* seq_ids, const int32_t* t0s,
                 int n_seqs, int layer, int loop, int q_len, int n_heads, int d, float scale,
                 void* stream) {
  if (n_seqs <= 0 || n_seqs > kMaxQSeqs) return -1;
  QRows rows;
  for (int b = 0; b < n_seqs; ++b) {
    rows.seq[b] = seq_ids[b];
    rows.t0[b] = t0s[b];
  }
  const int64_t total = (int64_t)n_seqs * q_len * n_heads * d;
  hipLaunchKernelGGL(fill_q_kernel, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)stream, dst,
                     dtype, seed, rows, (uint32_t)layer, (uint32_t)loop, n_seqs, q_len, n_heads, d,
                     scale);
  return (int)hipGetLastError();
}

int synth_fill_codes(void* dst, uint64_t seed, int tensor, int seq, int layer, int plane,
                     int n_heads, int d, int pos0, int n_pos, int bits, void* stream) {
  const int64_t total = (int64_t)n_pos * n_heads * d;
  if (total <= 0) return 0;
  hipLaunchKernelGGL(fill_codes_kernel, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)dst, seed, (uint32_t)tensor, (uint32_t)seq, (uint32_t)layer,
                     (uint32_t)plane, n_heads, d, pos0, n_pos, bits);
  return (int)hipGetLastError();
}

int synth_fill_meta(void* dst, uint64_t seed, int which, int seq, int layer, int plane,
                    int n_heads, int n_ch, int row0, int n_rows, int bits, void* stream) {
  const int64_t total = (int64_t)n_rows * n_heads * n_ch;
  if (total <= 0) return 0;
  const uint32_t ts = which == 0 ? kKScale : kVScale;
  const uint32_t tz = which == 0 ? kKZero : kVZero;
  hipLaunchKernelGGL(fill_meta_kernel, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)dst, seed, ts, tz, (uint32_t)seq, (uint32_t)layer, (uint32_t)plane,
                     n_heads, n_ch, row0, n_rows, bits);
  return (int)hipGetLastError();
}

}  // extern "C"
