// Shared pieces of the VALU attention kernels (decode, draft, cell near block):
// the plain-page tile geometry, per-lane partial dot products, quad accumulation
// and the online-softmax step of one 16-lane DPP row.
#pragma once
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "params.hpp"

namespace lkv {

template <typename T, int D>
struct DecodeTile {
  static constexpr int ES = sizeof(T) == 4 ? 4 : 2;
  static constexpr int E = D / 16;           // K channels and V channels per lane
  static constexpr int KB = E * ES;          // K bytes per lane per token: channels [li E, li E + E)
  static constexpr int VL = D * ES / 64;     // 16-byte V loads per lane per page
  static constexpr int VB = 16 * VL;         // V bytes per lane per page
  static constexpr int HEAD = kPage * D * ES;
};

// Channel of a lane's V element e.  Load j of lane li reads the 16 bytes at offset
// 256 j + 16 li of its quad: bf16 channels 32 j + 2 li and 32 j + 2 li + 1, fp32
// channel 16 j + li (four tokens each).
template <typename T>
__device__ __forceinline__ int vchan(int e, int li) {
  if constexpr (sizeof(T) == 4) return 16 * e + li;
  else return 32 * (e >> 1) + 2 * li + (e & 1);
}

// The lane's V block of one quad (quad_lane = quad base + 16 li).
template <typename T, int D>
__device__ __forceinline__ void load_vquad(Raw<DecodeTile<T, D>::VB>& v, const uint8_t* quad_lane) {
  load_stream_strided<DecodeTile<T, D>::VL>(v, quad_lane, 256);
}

// Partial score of one token: this lane's channels.
template <typename T, int D>
__device__ __forceinline__ float partial_dot(const Raw<DecodeTile<T, D>::KB>& k, const float* qf,
                                             const uint32_t* qw) {
  constexpr int E = D / 16;
  float s = 0.f;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int e = 0; e < E; ++e) s = fmaf(qf[e], __uint_as_float(k.w[e]), s);
  } else {
#pragma unroll
    for (int w = 0; w < E / 2; ++w) s = dot2_bf16(qw[w], k.w[w], s);
  }
  return s;
}

// o[e] += sum_k p[k] * v(channel e, token k) for this lane's quad block.
template <typename T, int D>
__device__ __forceinline__ void accum_quad(float* o, const Raw<DecodeTile<T, D>::VB>& v, const float* p) {
  constexpr int E = D / 16;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float a = o[e];
      a = fmaf(p[0], __uint_as_float(v.w[4 * e + 0]), a);
      a = fmaf(p[1], __uint_as_float(v.w[4 * e + 1]), a);
      a = fmaf(p[2], __uint_as_float(v.w[4 * e + 2]), a);
      a = fmaf(p[3], __uint_as_float(v.w[4 * e + 3]), a);
      o[e] = a;
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float a = o[e];
      a = fmaf(p[0], bf_lo(v.w[2 * e + 0]), a);
      a = fmaf(p[1], bf_hi(v.w[2 * e + 0]), a);
      a = fmaf(p[2], bf_lo(v.w[2 * e + 1]), a);
      a = fmaf(p[3], bf_hi(v.w[2 * e + 1]), a);
      o[e] = a;
    }
  }
}

// Per-token select between two quad blocks: token k taken from `b` where take_b[k].
// Tokens with zero[k] are cleared (keys beyond the sequence: their slots may hold NaN).
template <typename T, int D>
__device__ __forceinline__ void blend_quad(Raw<DecodeTile<T, D>::VB>& a, const Raw<DecodeTile<T, D>::VB>& b,
                                           const bool* take_b, const bool* zero) {
  constexpr int E = D / 16;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t x = take_b[k] ? b.w[4 * e + k] : a.w[4 * e + k];
        a.w[4 * e + k] = zero[k] ? 0u : x;
      }
  } else {
    const uint32_t sel01 = (take_b[0] ? 0x0000FFFFu : 0u) | (take_b[1] ? 0xFFFF0000u : 0u);
    const uint32_t sel23 = (take_b[2] ? 0x0000FFFFu : 0u) | (take_b[3] ? 0xFFFF0000u : 0u);
    const uint32_t keep01 = (zero[0] ? 0u : 0x0000FFFFu) | (zero[1] ? 0u : 0xFFFF0000u);
    const uint32_t keep23 = (zero[2] ? 0u : 0x0000FFFFu) | (zero[3] ? 0u : 0xFFFF0000u);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      a.w[2 * e + 0] = ((b.w[2 * e + 0] & sel01) | (a.w[2 * e + 0] & ~sel01)) & keep01;
      a.w[2 * e + 1] = ((b.w[2 * e + 1] & sel23) | (a.w[2 * e + 1] & ~sel23)) & keep23;
    }
  }
}

struct Softmax {
  float m;  // running max, base-2 units
  float l;
};

// Online softmax update of one DPP row with NT new base-2 logits x[].
template <int E, int NT>
__device__ __forceinline__ void softmax_step(Softmax& st, float* o, float* x) {
  float mn = st.m;
#pragma unroll
  for (int i = 0; i < NT; ++i) mn = fmaxf(mn, x[i]);
  const float mu = (mn == -INFINITY) ? 0.f : mn;
  const float alpha = fast_exp2(st.m - mu);
  float add = 0.f;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    x[i] = fast_exp2(x[i] - mu);
    add += x[i];
  }
  st.l = fmaf(st.l, alpha, add);
  st.m = mn;
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] *= alpha;
}

}  // namespace lkv
