// Device helpers for the CDNA4 (gfx950) attention kernels: bf16 bit conversions,
// 16-lane DPP reductions, vector loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct bf16 { uint16_t bits; };

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite values; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// bf16 pair dot product with fp32 accumulate (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the bitwise-same result.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// Eight 16-lane row sums at once, transposed.  Lane l of a DPP row holds in v[s] its
// partial value of item s ^ (l >> 1) (each lane keeps the eight items in its own order);
// lane l ends with the row sum of item l >> 1 (each sum held by two neighbouring lanes).
// Each step pairs a lane with one whose index differs in the next bits (mirror: l and
// 15 - l; half mirror: l and l ^ 7; quad permute: l ^ 2, then l ^ 1) and adds the
// partner's partial of the items it keeps; with that order of items the partner's
// partial sits in the same register in every lane, so the eight sums take 8 DPP adds and
// no selects.  Every item's partials are paired as in a plain butterfly.
__device__ __forceinline__ float row_sum16_t8(const float* v) {
  float a[4], c[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = v[k] + dpp<0x140>(v[7 - k]);
#pragma unroll
  for (int k = 0; k < 2; ++k) c[k] = a[k] + dpp<0x141>(a[3 - k]);
  const float e = c[0] + dpp<0x4E>(c[1]);
  return e + dpp<0xB1>(e);
}

// Value of lane n of the lane's DPP row (row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp<0x150 + N>(x);
}

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Online softmax with a lazy reference maximum, for accumulators that live in MFMA
// result registers (AGPRs), where a rescale costs a read, a multiply and a write per
// element: a column's reference maximum m moves only when a score passes it by more
// than kLazyLog2 (base-2 units).  Weights 2^(x - m) then stay below 2^kLazyLog2, the
// row sum and the accumulators keep using one m, so the softmax is the same, and once
// the first page has set m a wave almost never rescales (lazy_any skips it).
constexpr float kLazyLog2 = 8.f;

__device__ __forceinline__ bool lazy_any(bool grow) { return __builtin_amdgcn_ballot_w64(grow) != 0; }

// Raw dword loads of N bytes (N in {8, 12, 16, 32, 48, 64}); addresses are 4-byte aligned.
template <int NB>
struct Raw {
  uint32_t w[NB / 4];
};

template <int NB>
__device__ __forceinline__ void load_raw(Raw<NB>& r, const uint8_t* p) {
  static_assert(NB % 4 == 0, "dword multiple");
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + 16 * i);
      r.w[4 * i + 0] = v.x;
      r.w[4 * i + 1] = v.y;
      r.w[4 * i + 2] = v.z;
      r.w[4 * i + 3] = v.w;
    }
  } else if constexpr (NB == 12) {
    struct __attribute__((packed, aligned(4))) U3 { uint32_t x, y, z; };
    const U3 v = *reinterpret_cast<const U3*>(p);
    r.w[0] = v.x;
    r.w[1] = v.y;
    r.w[2] = v.z;
  } else if constexpr (NB == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) r.w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

// Streaming loads of page data that is read once per call.  They carry the
// nontemporal hint, which on gfx950 streams HBM noticeably faster than plain loads,
// but only where one load instruction of a wave covers whole 128-byte lines: lines
// fetched nontemporally are not kept for a later instruction that wants their rest.
// Same contract as load_raw.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int NB>
__device__ __forceinline__ void load_stream(Raw<NB>& r, const uint8_t* p) {
  static_assert(NB % 4 == 0, "dword multiple");
#pragma unroll
  for (int o = 0; o + 16 <= NB; o += 16) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + o));
    r.w[o / 4 + 0] = v.x;
    r.w[o / 4 + 1] = v.y;
    r.w[o / 4 + 2] = v.z;
    r.w[o / 4 + 3] = v.w;
  }
  if constexpr (NB % 16 >= 8) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p + (NB / 16) * 16));
    r.w[(NB / 16) * 4 + 0] = v.x;
    r.w[(NB / 16) * 4 + 1] = v.y;
  }
  if constexpr (NB % 8 == 4) r.w[NB / 4 - 1] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p + NB - 4));
}

// N loads of 16 bytes, `stride` bytes apart (nontemporal), into one register block.
template <int N>
__device__ __forceinline__ void load_stream_strided(Raw<16 * N>& r, const uint8_t* p, int stride) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + j * stride));
    r.w[4 * j + 0] = v.x;
    r.w[4 * j + 1] = v.y;
    r.w[4 * j + 2] = v.z;
    r.w[4 * j + 3] = v.w;
  }
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

template <typename T>
__device__ __forceinline__ void store_out(void* base, int64_t idx, float v);

template <>
__device__ __forceinline__ void store_out<float>(void* base, int64_t idx, float v) {
  reinterpret_cast<float*>(base)[idx] = v;
}

template <>
__device__ __forceinline__ void store_out<bf16>(void* base, int64_t idx, float v) {
  reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_bf16_bits(v);
}

template <typename T>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx);

template <>
__device__ __forceinline__ float load_elem<float>(const void* base, int64_t idx) {
  return reinterpret_cast<const float*>(base)[idx];
}

template <>
__device__ __forceinline__ float load_elem<bf16>(const void* base, int64_t idx) {
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[idx] << 16);
}

}  // namespace lkv
