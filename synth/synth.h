// Seeded synthetic inputs for loop-aware attention tests and benchmarks.
//
// This header holds input generation only: a counter-based hash, discrete
// normal and binomial draws, and exact rounding to bf16/fp16.  It contains no
// attention arithmetic.  The numpy implementation in synth/__init__.py follows
// the same definitions bit for bit; tests compare the two.
//
// Hash: the SplitMix64 output function (Steele, Lea and Flood, "Fast
// splittable pseudorandom number generators", OOPSLA 2014), applied in stages
// to fold a tensor's coordinates into a stream key, then once per counter.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace synth {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kMul1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kMul2 = 0x94D049BB133111EBull;
constexpr uint32_t kMask20 = (1u << 20) - 1u;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * kMul1;
  z = (z ^ (z >> 27)) * kMul2;
  return z ^ (z >> 31);
}

// Stream key of one (tensor, seq, layer, plane, head) row.
__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint32_t tensor, uint32_t seq,
                                               uint32_t layer, uint32_t plane, uint32_t head) {
  uint64_t k = mix64(seed + kGamma * (uint64_t)(1u + tensor));
  k = mix64(k + kGamma * (uint64_t)(1u + seq));
  k = mix64(k + kGamma * (uint64_t)(1u + layer));
  k = mix64(k + kGamma * (uint64_t)(1u + plane));
  k = mix64(k + kGamma * (uint64_t)(1u + head));
  return k;
}

__host__ __device__ inline uint64_t draw(uint64_t key, uint64_t counter) {
  return mix64(key + kGamma * (counter + 1ull));
}

// Irwin-Hall(12) normal on a 2^-20 grid: returns n with value n * 2^-20.
// |n| <= 6 * 2^20, so n * 2^-20 is exact in fp32.
__host__ __device__ inline int32_t normal20(uint64_t key, uint64_t elem) {
  uint64_t s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint64_t x = draw(key, 4ull * elem + (uint64_t)i);
    s += (x & kMask20) + ((x >> 20) & kMask20) + ((x >> 40) & kMask20);
  }
  return (int32_t)((int64_t)s - 6ll * (1ll << 20));
}

__host__ __device__ inline float normal_f32(uint64_t key, uint64_t elem) {
  return (float)normal20(key, elem) * (1.0f / 1048576.0f);
}

// Binomial(2^bits - 1, 1/2) code in [0, 2^bits - 1].
__host__ __device__ inline uint32_t binom_code(uint64_t key, uint64_t elem, int bits) {
  uint64_t x = draw(key, elem);
  uint32_t mask = (1u << ((1 << bits) - 1)) - 1u;
  return (uint32_t)__builtin_popcount((uint32_t)x & mask);
}

__host__ __device__ inline uint32_t f32_bits(float f) {
  union { float f; uint32_t u; } c; c.f = f; return c.u;
}
__host__ __device__ inline float bits_f32(uint32_t u) {
  union { float f; uint32_t u; } c; c.u = u; return c.f;
}
__host__ __device__ inline uint64_t f64_bits(double d) {
  union { double d; uint64_t u; } c; c.d = d; return c.u;
}
__host__ __device__ inline double bits_f64(uint64_t u) {
  union { double d; uint64_t u; } c; c.u = u; return c.d;
}

// fp32 -> bf16, round to nearest even (finite inputs).
__host__ __device__ inline uint16_t bf16_from_f32(float f) {
  uint32_t u = f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 with a single rounding to nearest even (finite inputs within
// the fp32 normal range).  Rounds the fp64 significand at bf16's last bit.
__host__ __device__ inline uint16_t bf16_from_f64(double d) {
  uint64_t u = f64_bits(d);
  const uint64_t lsb = (u >> 45) & 1ull;
  u += ((1ull << 44) - 1ull) + lsb;
  u &= ~((1ull << 45) - 1ull);
  return (uint16_t)(f32_bits((float)bits_f64(u)) >> 16);
}

__host__ __device__ inline float f32_from_bf16(uint16_t h) { return bits_f32((uint32_t)h << 16); }

// fp32 -> fp16, round to nearest even, including subnormals and overflow.
__host__ __device__ inline uint16_t f16_from_f32(float f) {
  uint32_t u = f32_bits(f);
  const uint32_t sign = (u >> 16) & 0x8000u;
  u &= 0x7FFFFFFFu;
  if (u >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (u > 0x7F800000u ? 0x200u : 0u));
  const uint32_t e = u >> 23;
  uint32_t h, rem, half;
  if (e < 113u) {  // below 2^-14: fp16 subnormal or zero
    const uint32_t shift = 126u - e;
    if (shift > 31u) return (uint16_t)sign;
    const uint32_t m = (u & 0x7FFFFFu) | 0x800000u;
    h = m >> shift;
    rem = m & ((1u << shift) - 1u);
    half = 1u << (shift - 1u);
  } else {
    h = ((e - 112u) << 10) | ((u & 0x7FFFFFu) >> 13);
    rem = u & 0x1FFFu;
    half = 0x1000u;
  }
  if (rem > half || (rem == half && (h & 1u))) h += 1u;
  if (h > 0x7C00u) h = 0x7C00u;
  return (uint16_t)(sign | h);
}

// Tensor ids of the synthetic streams.
enum Tensor : uint32_t {
  kK = 1, kV = 2, kQ = 3, kKNoise = 4, kVNoise = 5,
  kKCode = 6, kVCode = 7, kKScale = 8, kKZero = 9, kVScale = 10, kVZero = 11,
  kDraftK = 12, kDraftV = 13, kPlan = 14, kPerm = 15,
};

}  // namespace synth
