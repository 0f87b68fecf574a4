// LoopKV-style quantised cells: packed code pages and the cell attention kernel.
//
// Code page (32 far-history tokens of one (seq, layer, loop) cell, all KV heads;
// head_dim 128).  Per head, INT4 (40 * D bytes = 160 B per token-head: 4-bit K and
// V codes plus fp16 scale/zero per 32 elements, LoopKV page App. C):
//   [0,    4D)  K meta   [channel][scale, zero] fp16, per channel over the page
//   [4D,  20D)  K codes  4-bit, lane-major: [half][g][li][4 slots][8 nibbles]; slot
//                        i ^ (li >> 1) holds token 4 i + g (kslot)
//   [20D, 28D)  V hi     2-bit hi = c >> 2, lane-major: [g][li][8 tokens][16 bits]
//   [28D, 36D)  V lo     2-bit lo = c & 3, token-major: [token][li][16 bits]
//   [36D, 40D)  V meta   [g][group][8 tokens][scale, zero] fp16, per token and 32 channels
// INT2 (24 * D bytes): K meta [0,4D), K codes [4D,12D) as V hi, V codes [12D,20D)
// as V hi, V meta [20D,24D).  Lane (g, li) of a DPP row owns channels 8li..8li+7
// and tokens g, g+4, ..., g+28 of the page, so its K codes, V hi and V meta are
// contiguous 16-32 B runs; V lo is token-major so that a cold token's 32-byte lo
// row (one token-head) is never requested at all (LoopKV page, Sec. 3.3).
//
// Bit order inside a lane's 16-bit word of 2-bit values (its 8 channels c):
// hi crumbs sit at crumb 2c + 1 (c < 4) or 2(c - 4) (c >= 4), lo and INT2 crumbs
// at crumb 2c (c < 4) or 2(c - 4) + 1 (c >= 4).  Then x | x << 18 puts hi_c at
// bits 2-3 of nibble c and y | y << 14 puts lo_c at bits 0-1 of nibble c, so one
// bitfield insert yields the eight 4-bit codes 4 hi + lo of a hot token.  K codes are
// plain nibbles (nibble c = channel c).  Nibble words and INT2 words reach the
// arithmetic as exact fp16 pairs (offset + code) with one mask-and-exponent
// instruction per pair (int4_pairs_f16, int2_pairs_f16).
#include <hip/hip_runtime.h>

#include "attn_common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "params.hpp"

namespace lkv {

uint64_t code_page_bytes(int hkv, int head_dim, int bits) {
  return (uint64_t)hkv * (bits == 4 ? 40 : 24) * head_dim;
}

// Crumb positions of channel c (0..7) in a lane's 16-bit V word (see the layout above).
__host__ __device__ __forceinline__ int hi_crumb(int c) { return c < 4 ? 2 * c + 1 : 2 * (c - 4); }
__host__ __device__ __forceinline__ int lo_crumb(int c) { return c < 4 ? 2 * c : 2 * (c - 4) + 1; }

// Key slot of token 4 i + g in lane li's K code words: i ^ (li >> 1), the order in which
// the transposed 16-lane score sums take a lane's eight tokens without selects.
__host__ __device__ __forceinline__ int kslot(int i, int li) { return i ^ (li >> 1); }

// Byte offsets inside one head's slice of a code page (d = 128).
__host__ __device__ constexpr uint64_t code_head_bytes(int bits) { return (uint64_t)(bits == 4 ? 40 : 24) * 128; }
__host__ __device__ constexpr uint64_t vcode_offset(int bits) { return (bits == 4 ? 20 : 12) * 128; }
__host__ __device__ constexpr uint64_t vmeta_offset(int bits) { return (bits == 4 ? 36 : 20) * 128; }

// Store lane li's 8 channels of token tok (codes kin[0..7], vin[0..7]) into the head
// slice hb.  Lanes li < 4 also store the token's V metadata of group li (vm_src:
// scale, zero), tokens tok < 8 the K metadata of channel 16 tok + li (km_src).
__device__ __forceinline__ void pack_item(uint8_t* hb, int bits, int tok, int li, const uint8_t* kin,
                                          const uint8_t* vin, const uint16_t* vm_src, const uint16_t* km_src) {
  constexpr int D = 128;
  const int g = tok & 3, i = tok >> 2;
  if (bits == 4) {
    uint32_t kw = 0, vhi = 0, vlo = 0;
    for (int c = 0; c < 8; ++c) {
      kw |= (uint32_t)(kin[c] & 15u) << (4 * c);
      vhi |= (uint32_t)((vin[c] >> 2) & 3u) << (2 * hi_crumb(c));
      vlo |= (uint32_t)(vin[c] & 3u) << (2 * lo_crumb(c));
    }
    const int ks = kslot(i, li), hh = ks >> 2, ii = ks & 3;
    *reinterpret_cast<uint32_t*>(hb + 4 * D + hh * 1024 + (g * 16 + li) * 16 + ii * 4) = kw;
    *reinterpret_cast<uint16_t*>(hb + 20 * D + (g * 16 + li) * 16 + i * 2) = (uint16_t)vhi;
    *reinterpret_cast<uint16_t*>(hb + 28 * D + tok * 32 + li * 2) = (uint16_t)vlo;
  } else {
    uint32_t kw = 0, vw = 0;
    for (int c = 0; c < 8; ++c) {
      kw |= (uint32_t)(kin[c] & 3u) << (2 * lo_crumb(c));
      vw |= (uint32_t)(vin[c] & 3u) << (2 * lo_crumb(c));
    }
    *reinterpret_cast<uint16_t*>(hb + 4 * D + (g * 16 + li) * 16 + kslot(i, li) * 2) = (uint16_t)kw;
    *reinterpret_cast<uint16_t*>(hb + 12 * D + (g * 16 + li) * 16 + i * 2) = (uint16_t)vw;
  }
  if (li < 4) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(hb + vmeta_offset(bits) + ((g * 4 + li) * 8 + i) * 4);
    dst[0] = vm_src[0];
    dst[1] = vm_src[1];
  }
  if (tok < 8) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(hb + (tok * 16 + li) * 4);
    dst[0] = km_src[0];
    dst[1] = km_src[1];
  }
}

// Inverse of pack_item: read lane li's 8 channels of token tok back into plain codes.
__device__ __forceinline__ void unpack_item(const uint8_t* hb, int bits, int tok, int li, uint8_t* kout,
                                            uint8_t* vout, uint16_t* vm_dst, uint16_t* km_dst) {
  constexpr int D = 128;
  const int g = tok & 3, i = tok >> 2;
  if (bits == 4) {
    const int ks = kslot(i, li), hh = ks >> 2, ii = ks & 3;
    const uint32_t kw = *reinterpret_cast<const uint32_t*>(hb + 4 * D + hh * 1024 + (g * 16 + li) * 16 + ii * 4);
    const uint32_t vhi = *reinterpret_cast<const uint16_t*>(hb + 20 * D + (g * 16 + li) * 16 + i * 2);
    const uint32_t vlo = *reinterpret_cast<const uint16_t*>(hb + 28 * D + tok * 32 + li * 2);
    for (int c = 0; c < 8; ++c) {
      kout[c] = (uint8_t)((kw >> (4 * c)) & 15u);
      vout[c] = (uint8_t)((((vhi >> (2 * hi_crumb(c))) & 3u) << 2) | ((vlo >> (2 * lo_crumb(c))) & 3u));
    }
  } else {
    const uint32_t kw = *reinterpret_cast<const uint16_t*>(hb + 4 * D + (g * 16 + li) * 16 + kslot(i, li) * 2);
    const uint32_t vw = *reinterpret_cast<const uint16_t*>(hb + 12 * D + (g * 16 + li) * 16 + i * 2);
    for (int c = 0; c < 8; ++c) {
      kout[c] = (uint8_t)((kw >> (2 * lo_crumb(c))) & 3u);
      vout[c] = (uint8_t)((vw >> (2 * lo_crumb(c))) & 3u);
    }
  }
  if (li < 4) {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(hb + vmeta_offset(bits) + ((g * 4 + li) * 8 + i) * 4);
    vm_dst[0] = src[0];
    vm_dst[1] = src[1];
  }
  if (tok < 8) {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(hb + (tok * 16 + li) * 4);
    km_dst[0] = src[0];
    km_dst[1] = src[1];
  }
}

// One thread per (head, token, lane li) of one page (blockIdx.y = page of the batch):
// packs that lane's 8 channels of one token from the logical arrays.
__global__ __launch_bounds__(256) void pack_codes_kernel(const PackParams p) {
  constexpr int D = 128;
  const int pi = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int hkv = p.hkv;
  if (idx >= hkv * kCodePage * 16 || pi >= p.n_pages) return;
  const int li = idx & 15, tok = (idx >> 4) & 31, h = idx >> 9;
  uint8_t* hb = p.arena + (uint64_t)p.phys[pi] * p.page_bytes + (uint64_t)h * code_head_bytes(p.bits);
  const int64_t row = ((int64_t)pi * kCodePage + tok) * hkv + h;
  pack_item(hb, p.bits, tok, li, p.k_codes + row * D + 8 * li, p.v_codes + row * D + 8 * li,
            p.v_meta + (row * (D / 32) + (li & 3)) * 2,
            p.k_meta + (((int64_t)pi * hkv + h) * D + ((tok & 7) * 16 + li)) * 2);
}

// Inverse: one thread per (head, token, lane li) of one page, into the logical arrays.
__global__ __launch_bounds__(256) void read_codes_kernel(const PackParams p, uint8_t* k_codes, uint16_t* k_meta,
                                                         uint8_t* v_codes, uint16_t* v_meta) {
  constexpr int D = 128;
  const int pi = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int hkv = p.hkv;
  if (idx >= hkv * kCodePage * 16 || pi >= p.n_pages) return;
  const int li = idx & 15, tok = (idx >> 4) & 31, h = idx >> 9;
  const uint8_t* hb = p.arena + (uint64_t)p.phys[pi] * p.page_bytes + (uint64_t)h * code_head_bytes(p.bits);
  const int64_t row = ((int64_t)pi * kCodePage + tok) * hkv + h;
  unpack_item(hb, p.bits, tok, li, k_codes + row * D + 8 * li, v_codes + row * D + 8 * li,
              v_meta + (row * (D / 32) + (li & 3)) * 2, k_meta + (((int64_t)pi * hkv + h) * D + ((tok & 7) * 16 + li)) * 2);
}

// The window-exit codec (LoopKV page, Sec. 3.1 and 3.3; KIVI-style): one workgroup
// of 128 threads per (page, head) encodes 32 tokens of exact bf16 keys and values.
// Keys: one group per channel over the page's valid tokens; values: one group per
// token and 32 channels.  Per group: mn, mx; scale = (mx - mn) / (2^b - 1) in fp32
// (IEEE division), zero = mn, both rounded to fp16 (nearest even); a value's code is
// rint((x - zero16) / scale16) clamped to [0, 2^b - 1] (0 when scale16 = 0), each
// operation rounded in fp32.  Tokens past n_valid of the last page get code 0 and
// zero metadata.  The codes go through LDS into the page's packed layout.
__device__ __forceinline__ float bf16_bits_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ void encode_group(const uint16_t* x, int n, int stride, int levels, uint8_t* c,
                                             int cstride, uint16_t* meta) {
  float mn = bf16_bits_f32(x[0]), mx = mn;
  for (int i = 1; i < n; ++i) {
    const float v = bf16_bits_f32(x[(int64_t)i * stride]);
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  const float sigma = (mx - mn) / (float)levels;  // correctly rounded (HIP's fp32 division)
  const _Float16 s16 = (_Float16)sigma, z16 = (_Float16)mn;  // v_cvt_f16_f32: nearest even
  const float sf = (float)s16, zf = (float)z16;
  for (int i = 0; i < n; ++i) {
    float q = 0.f;
    if (sf != 0.f) {
      q = rintf((bf16_bits_f32(x[(int64_t)i * stride]) - zf) / sf);
      q = fminf(fmaxf(q, 0.f), (float)levels);
    }
    c[i * cstride] = (uint8_t)q;
  }
  meta[0] = __builtin_bit_cast(uint16_t, s16);
  meta[1] = __builtin_bit_cast(uint16_t, z16);
}

__global__ __launch_bounds__(128) void encode_pages_kernel(const EncodeParams p) {
  constexpr int D = 128;
  const int pi = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (pi >= p.n_pages || h >= p.hkv) return;  // uniform per workgroup
  const int n = pi == p.n_pages - 1 ? p.n_valid_last : kCodePage;
  const int levels = (1 << p.bits) - 1;
  __shared__ uint8_t kc[kCodePage][D], vc[kCodePage][D];
  __shared__ uint16_t km[D][2], vm[kCodePage][4][2];
  // the page's exact keys and values of head h, token-major, staged in LDS (thread = channel)
  __shared__ uint16_t kx[kCodePage][D], vx[kCodePage][D];
  for (int t = 0; t < n; ++t) {
    if (p.tab_plain) {
      // plain page layout: K block [head][token][channel]; V block [head][quad][channel][i],
      // entry i of quad g = token 4 i + g
      const int j = p.pos0 + pi * kCodePage + t, s = j % kPage;
      const uint8_t* base = p.pool + (uint64_t)p.tab_plain[j / kPage] * p.plain_page_bytes;
      const uint64_t head = (uint64_t)kPage * D * 2;
      kx[t][tid] = *reinterpret_cast<const uint16_t*>(base + h * head + ((uint64_t)s * D + tid) * 2);
      vx[t][tid] = *reinterpret_cast<const uint16_t*>(base + (p.hkv + h) * head +
                                                      (((uint64_t)(s & 3) * D + tid) * kQuad + (s >> 2)) * 2);
    } else {
      const int64_t row = ((int64_t)pi * kCodePage + t) * p.hkv + h;
      kx[t][tid] = p.k[row * D + tid];
      vx[t][tid] = p.v[row * D + tid];
    }
  }
  __syncthreads();
  // keys: thread = channel
  encode_group(&kx[0][tid], n, D, levels, &kc[0][tid], D, km[tid]);
  for (int t = n; t < kCodePage; ++t) kc[t][tid] = 0;
  // values: thread = (token, 32-channel group)
  {
    const int t = tid >> 2, grp = tid & 3;
    if (t < n) {
      encode_group(&vx[t][32 * grp], 32, 1, levels, &vc[t][32 * grp], 1, vm[t][grp]);
    } else {
      for (int c = 0; c < 32; ++c) vc[t][32 * grp + c] = 0;
      vm[t][grp][0] = 0;
      vm[t][grp][1] = 0;
    }
  }
  __syncthreads();
  uint8_t* hb = p.arena + (uint64_t)p.phys[pi] * p.page_bytes + (uint64_t)h * code_head_bytes(p.bits);
  for (int it = tid; it < kCodePage * 16; it += 128) {
    const int tok = it >> 4, li = it & 15;
    pack_item(hb, p.bits, tok, li, &kc[tok][8 * li], &vc[tok][8 * li], vm[tok][li & 3], km[(tok & 7) * 16 + li]);
  }
}

hipError_t launch_encode_pages(const EncodeParams& p, int head_dim, hipStream_t s) {
  if (head_dim != 128 || p.n_pages < 1 || p.n_pages > 64 || p.n_valid_last < 1 || p.n_valid_last > kCodePage ||
      (p.bits != 4 && p.bits != 2))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(encode_pages_kernel, dim3(p.n_pages, p.hkv), dim3(128), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_read_codes(const PackParams& p, int head_dim, void* k_codes, void* k_meta, void* v_codes,
                             void* v_meta, hipStream_t s) {
  if (head_dim != 128 || p.n_pages < 1 || p.n_pages > 64) return hipErrorInvalidValue;
  const int n = p.hkv * kCodePage * 16;
  hipLaunchKernelGGL(read_codes_kernel, dim3((n + 255) / 256, p.n_pages), dim3(256), 0, s, p,
                     reinterpret_cast<uint8_t*>(k_codes), reinterpret_cast<uint16_t*>(k_meta),
                     reinterpret_cast<uint8_t*>(v_codes), reinterpret_cast<uint16_t*>(v_meta));
  return hipGetLastError();
}

hipError_t launch_pack_codes(const PackParams& p, int head_dim, hipStream_t s) {
  if (head_dim != 128 || p.n_pages < 1 || p.n_pages > 64) return hipErrorInvalidValue;
  const int n = p.hkv * kCodePage * 16;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((n + 255) / 256, p.n_pages), dim3(256), 0, s, p);
  return hipGetLastError();
}

// max(x, its DPP partner) as v_med3_f32(x, y, +inf): for the non-NaN scores it sees this is
// the larger one, and unlike fmaxf it does not quiet its DPP-moved input first (one VALU
// instruction fewer per step).  The +inf comes through an empty asm so that the compiler
// does not turn the median back into a max.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float x) {
  float inf = __builtin_inff();
  asm("" : "+s"(inf));
  return __builtin_amdgcn_fmed3f(x, dpp<CTRL>(x), inf);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// V codes 4 hi + lo of two tokens a, b from their crumb words: hi = H (a in the low half,
// b in the high half), lo = L (same).  Channels c < 4 have hi at odd and lo at even crumbs
// (crumbs 2c + 1 and 2c), so one bit-field select of the odd crumbs of H and the even
// crumbs of L gives nibble c = 4 hi_c + lo_c in each half; channels c >= 4 have them the
// other way round (hi at crumb 2(c - 4), lo at 2(c - 4) + 1), and H << 2, L >> 2 move
// them to the same places (a crumb that crosses into the other half lands in the part the
// select drops).  Each half of the two results holds the nibbles of channels 0-3 resp.
// 4-7 of its token.
__device__ __forceinline__ uint32_t vcodes_lo4(uint32_t H, uint32_t L) { return (H & 0xCCCCCCCCu) | (L & 0x33333333u); }
__device__ __forceinline__ uint32_t vcodes_hi4(uint32_t H, uint32_t L) {
  return ((H << 2) & 0xCCCCCCCCu) | ((L >> 2) & 0x33333333u);
}

__device__ __forceinline__ uint32_t or4(uint32_t v) {
  v |= (uint32_t)__shfl_xor((int)v, 16);
  v |= (uint32_t)__shfl_xor((int)v, 32);
  return v;
}

// INT2 codes as fp16 pairs.  A lane's 32-bit word of INT2 codes holds two tokens, one
// per 16-bit half, with channel c's crumb at bit crumb_bit(c) of each half.  A crumb at
// bits 4-5, 6-7 or 8-9 of a half lies in an fp16 mantissa whose unit is 1 for the
// exponents of 64, 16 and 4: masking the word to that crumb in both halves and ORing
// in the exponent gives the exact pair (off + code of the low token, off + code of the
// high token), one v_and_or_b32.  Three channels already sit there; w >> 6 and w << 4
// bring the other five there, so a word takes 2 shifts and 8 v_and_or_b32 for its 16
// codes.  The offsets come off once (the sum of q' off for keys, the sum of the weights
// for values).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int crumb_bit(int c) { return 2 * (c < 4 ? 2 * c : 2 * (c - 4) + 1); }

// fp16 offset of channel c's pair (64, 16 or 4 by the bit its crumb is brought to)
__host__ __device__ constexpr float int2_off(int c) {
  return (c == 0 || c == 1 || c == 6) ? 64.f : (c == 2 || c == 7) ? 4.f : 16.f;
}

// v_and_or_b32 (x & mask) | base, written as an instruction because the compiler splits
// it into an and and an or.  Inline asm is opaque to the compiler's hazard checks: it only
// takes code words (loaded, shifted or combined by bitwise ops) and constants, never the
// result of a transcendental op (v_exp and the like), which a dependent VALU op on gfx950
// may read only after a wait state.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t base) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(base));
  return r;
}

// The eight fp16 pairs of a word (pair c: channel c of the low and the high token).
__device__ __forceinline__ void int2_pairs_f16(uint32_t w, uint32_t b64, uint32_t b16, uint32_t b4, uint32_t* pr) {
  const uint32_t x1 = w >> 6, x2 = w << 4;
  pr[0] = and_or(x2, 0x00300030u, b64);  // bits 0-1 -> 4-5
  pr[1] = and_or(w, 0x00300030u, b64);   // bits 4-5
  pr[2] = and_or(w, 0x03000300u, b4);    // bits 8-9
  pr[3] = and_or(x1, 0x00C000C0u, b16);  // bits 12-13 -> 6-7
  pr[4] = and_or(x2, 0x00C000C0u, b16);  // bits 2-3 -> 6-7
  pr[5] = and_or(w, 0x00C000C0u, b16);   // bits 6-7
  pr[6] = and_or(x1, 0x00300030u, b64);  // bits 10-11 -> 4-5
  pr[7] = and_or(x1, 0x03000300u, b4);   // bits 14-15 -> 8-9
}

// INT4 codes as fp16 pairs.  A word of 8 nibbles holds nibbles k and k + 4 exactly 16 bits
// apart, so the same mask-and-exponent step gives the pair (off + nibble k, off + nibble
// k + 4): nibbles at bits 4-7 are units of fp16 64, at bits 6-9 units of fp16 16.  In a K
// code word nibble c is channel c of one token, so pair k is channels (k, k + 4); in the V
// words of vcodes_lo4 / vcodes_hi4 pair k is one channel of two tokens.  Pairs 0 and 1 take
// offset 64, 2 and 3 offset 16; three shifts and four v_and_or_b32 per word of eight codes.
__host__ __device__ constexpr float int4_off(int c) { return (c & 3) < 2 ? 64.f : 16.f; }

__device__ __forceinline__ void int4_pairs_f16(uint32_t w, uint32_t b64, uint32_t b16, uint32_t* pr) {
  pr[0] = and_or(w << 4, 0x00F000F0u, b64);  // nibbles 0, 4 -> bits 4-7 of each half
  pr[1] = and_or(w, 0x00F000F0u, b64);       // nibbles 1, 5 at bits 4-7
  pr[2] = and_or(w >> 2, 0x03C003C0u, b16);  // nibbles 2, 6 -> bits 6-9
  pr[3] = and_or(w >> 6, 0x03C003C0u, b16);  // nibbles 3, 7 -> bits 6-9
}

// A code page's head slice as a buffer resource (base and size in scalar registers): each
// load then takes the page in the resource and a 32-bit lane offset, loop-invariant per
// load site, instead of a 64-bit address pair per lane; loads past the slice return 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t slice_rsrc(const uint8_t* hb, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(hb), 0, (int)bytes, 0x00020000);
}

// NB bytes (16 or 32) at byte offset off of the resource; NT: nontemporal (whole lines only)
// (SOFF, a constant, goes in the instruction's scalar offset)
template <int NB, bool NT, int SOFF = 0>
__device__ __forceinline__ void buf_load(Raw<NB>& r, rsrc_t rs, uint32_t off) {
#pragma unroll
  for (int o = 0; o < NB; o += 16) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, SOFF + o, NT ? 2 : 0);
    r.w[o / 4 + 0] = v.x;
    r.w[o / 4 + 1] = v.y;
    r.w[o / 4 + 2] = v.z;
    r.w[o / 4 + 3] = v.w;
  }
}

__device__ __forceinline__ float f16_lo_f32(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi_f32(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// One launch per cell: grid.x = n_splits far blocks + 1 near block.
//   near part (near block): exact bf16 attention over the sink [0, sink) and the tail
//     [L - tail, L) of the cell's own loop (LoopKV page, Sec. 3.2: sink and window
//     stay the cell's own and exact);
//   far part (every block, the near block after its near part, so that no block idles
//     once its near work is done): a share of the code pages of the cell's source (own
//     codes, or the final loop's for a shared cell).  Per page the K scale is folded into q
//     and q.z into a bias (LoopKV page, App. E), so a score is bias + sum q'_c c_jc.
//     The seed m0 is the largest sink score, recomputed by every block from the
//     sink keys (no wait on another block).  Hot test of a far token: the fixed
//     rule s_j >= m0 - offset, or the page's own rule s_j >= max(m, m0) - tau ln 2
//     with m the block's running maximum over its far pages so far (RUNNING).
//     V: hot tokens read both bit planes (4 hi + lo), cold tokens only hi and take
//     the bucket midpoint 4 hi + 1.5; the per-token V scale and zero fold into the
//     weight p_j (LoopKV page, Sec. 3.3, App. E Alg. 1).
// Each DPP row keeps its own online softmax; partials go to the workspace and
// the LSE merge kernel combines them.  In the far part a page's eight token scores
// of a row are summed transposed, so that lanes 2t and 2t + 1 hold token t's score:
// each lane takes one exponential, and the weights and hot bits reach the whole row
// by lane broadcasts.
template <int WAVES, bool TRACE, int BITS, bool RUNNING>
// Five waves per SIMD (96 VGPRs): the fixed-rule loops hold one page's state while the next
// page's loads are in flight (INT4: while its scores are computed), the running rule a page's
// scores across a barrier.  The traced variants, for tests, are left unconstrained.
__global__ __launch_bounds__(WAVES * 64, TRACE ? 1 : 5) void cell_kernel(const CellParams p) {
  constexpr int D = 128, E = 8;
  constexpr uint64_t HEADB = (uint64_t)kPage * D * 2;  // bf16 (page, head) slice
  const int part = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int hk = h / (p.hq / p.hkv);
  const int slot = p.slot[b];
  const int L = p.len[b];
  const int n_far = L - p.sink - p.tail;
  const int tail_lo = L - p.tail;

  // q: this lane's channels 8 li .. 8 li + 7, as bf16 pairs (dot2; converted per page in the
  // far blocks)
  uint32_t qw[E / 2];
  {
    Raw<16> r;
    load_raw<16>(r, reinterpret_cast<const uint8_t*>(p.q) + (((int64_t)b * p.hq + h) * D + li * E) * 2);
#pragma unroll
    for (int x = 0; x < 4; ++x) qw[x] = r.w[x];
  }
  const int32_t* tab_near = p.tab_near + (int64_t)slot * p.ring_near;
  const uint64_t koff = (uint64_t)hk * HEADB + (uint64_t)li * 16;
  const uint64_t voff = (uint64_t)p.hkv * HEADB + (uint64_t)hk * HEADB + (uint64_t)g * (kQuad * D * 2) + li * 16;

  Softmax st{-INFINITY, 0.f};
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  float zacc = 0.f;
  float wacc = 0.f;  // far part: the running sum of the V weights (fp16-rounded), rescaled like o

  // Row states of the block's waves for the final merge: far rows [0, 4 WAVES), and in the
  // near block its near rows [4 WAVES, 8 WAVES).
  __shared__ float sm_o[WAVES * 8][D];
  __shared__ float sm_m[WAVES * 8], sm_l[WAVES * 8];
  const int r = w * 4 + g;
  const bool near_block = part == p.n_splits;

  if (near_block) {
    // ---------------- near part (the near block only): sink and tail, bf16, own loop
    const int np_sink = (p.sink + kPage - 1) / kPage;
    const int tp0 = max(np_sink, tail_lo / kPage), tp1 = (L - 1) / kPage;
    const int count = np_sink + (p.tail > 0 ? max(0, tp1 - tp0 + 1) : 0);
    for (int k = w; k < count; k += WAVES) {
      const int pg = k < np_sink ? k : tp0 + (k - np_sink);
      const uint8_t* base = p.pool + (uint64_t)tab_near[pg] * p.page_bytes;
      Raw<16> kr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) load_stream<16>(kr[i], base + koff + (uint64_t)(4 * i + g) * (D * 2));
      Raw<64> vr;
      load_vquad<bf16, D>(vr, base + voff);
      bool zero[4], none[4] = {false, false, false, false};
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = pg * kPage + 4 * i + g;
        const bool valid = j < p.sink || (j >= tail_lo && j < L);
        zero[i] = !valid;
        float s = 0.f;
#pragma unroll
        for (int x2 = 0; x2 < 4; ++x2) s = dot2_bf16(qw[x2], kr[i].w[x2], s);
        s = row_sum16(s) * p.scale_log2;
        x[i] = valid ? s : -INFINITY;
      }
      blend_quad<bf16, D>(vr, vr, none, zero);
      softmax_step<E, 4>(st, o, x);
      accum_quad<bf16, D>(o, vr, x);
    }
    // park the near row states and start the far part from an empty state
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sm_o[WAVES * 4 + r][vchan<bf16>(e, li)] = o[e];
      o[e] = 0.f;
    }
    if (li == 0) {
      sm_m[WAVES * 4 + r] = st.m;
      sm_l[WAVES * 4 + r] = st.l;
    }
    st = Softmax{-INFINITY, 0.f};
  }
  {
    // ---------------- far part (every block: n_splits far blocks and the near block split
    // the code pages, the near block's share shorter by its near work)
    // seed m0: largest exact sink score (natural-log units)
    float m0 = -INFINITY;
    for (int sp = 0; sp * kPage < p.sink; ++sp) {  // sink pages (the page's own rule uses 32 sink keys)
      const uint8_t* base = p.pool + (uint64_t)tab_near[sp] * p.page_bytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * g + i;
        if (sp * kPage + j < p.sink) {  // uniform per DPP row
          Raw<16> kr;
          load_raw<16>(kr, base + koff + (uint64_t)j * (D * 2));
          float s = 0.f;
#pragma unroll
          for (int x2 = 0; x2 < 4; ++x2) s = dot2_bf16(qw[x2], kr.w[x2], s);
          m0 = fmaxf(m0, row_sum16(s) * p.scale);
        }
      }
    }
    m0 = fmaxf(m0, __shfl_xor(m0, 16));
    m0 = fmaxf(m0, __shfl_xor(m0, 32));
    const uint32_t b64 = 0x54005400u, b16 = 0x4C004C00u, b4 = 0x44004400u;  // fp16 64, 16, 4 in both halves
    constexpr float kLog2e = 1.4426950408889634f;
    // headroom of a row's far reference over the page maximum that set it (base-2 units):
    // the largest weight of that page is 2^-2, and later pages rescale only on a new
    // maximum more than that above it
    constexpr float kFarHeadroom = 2.f;
    constexpr bool masked = BITS == 4;  // INT4 and shared cells carry the hi / lo bit planes
    // The code-page table in the constant address space: the kernel never writes it, so its
    // entries stay scalar loads also after a barrier (which a plain global pointer's loads do
    // not: any barrier could order another workgroup's write before them)
    typedef const int32_t __attribute__((address_space(4)))* const_tab_t;
    const const_tab_t tab_code = (const_tab_t)(p.tab_code + (int64_t)slot * p.code_ring);
    constexpr uint64_t head_bytes = (uint64_t)(BITS == 4 ? 40 : 24) * D;
    // The n_splits + 1 blocks of a row take equal shares of the code pages plus the near
    // work, counted as the code pages of the same bytes (sink + tail tokens of bf16 K and V);
    // the near block's far share is its share less that.  Under the running rule the hot
    // sets depend on how the pages are cut into runs (each far split keeps its own running
    // maximum), so there the n_splits far blocks take equal shares and the near block none.
    const int n_cp = (n_far + kCodePage - 1) / kCodePage;
    int c0, c1;
    if constexpr (RUNNING && masked) {
      c0 = near_block ? n_cp : (int)((int64_t)part * n_cp / p.n_splits);
      c1 = near_block ? n_cp : (int)((int64_t)(part + 1) * n_cp / p.n_splits);
    } else {
      const int64_t near_eq = ((int64_t)(p.sink + p.tail) * 4 * D + (int64_t)head_bytes - 1) / (int64_t)head_bytes;
      const int64_t total = n_cp + near_eq;
      c0 = (int)min((int64_t)n_cp, (int64_t)part * total / (p.n_splits + 1));
      c1 = near_block ? n_cp : (int)min((int64_t)n_cp, (int64_t)(part + 1) * total / (p.n_splits + 1));
    }
    constexpr uint64_t vcode_off = BITS == 4 ? 20 * D : 12 * D;
    constexpr uint64_t vmeta_off = BITS == 4 ? 36 * D : 20 * D;
    // INT2 cells: the query for the far keys as an fp16 pair per channel c, (-off_c q_c 2^s,
    // q_c 2^s), where off_c is the offset of the channel's code pairs and 2^s puts the row's
    // largest |q_c| in [512, 1024).  Both elements are exact fp16 values (a bf16 query has 8
    // significant bits, and 64 x 1024 stays below the fp16 maximum); only channels more than
    // 2^23 below the largest fall to fp16 subnormals, where their products are under the fp32
    // rounding of the score.  One v_dot2 of the pair with the page's (sigma_c, z_c) metadata
    // adds both q_c z_c and the code offset's share to a page's bias, and the scores, 2^s too
    // large, come back through the scale.  (INT4 cells keep the bf16 query: their loops hold
    // 96 VGPRs, and with the pairs they spilled.)
    uint32_t qp[E] = {};
    float scale2 = p.scale_log2;
    if constexpr (BITS == 2) {
      float qa = 0.f;
#pragma unroll
      for (int x = 0; x < E / 2; ++x) qa = fmaxf(qa, fmaxf(fabsf(bf_lo(qw[x])), fabsf(bf_hi(qw[x]))));
      qa = row_max16(qa);  // the 16 lanes of a DPP row hold the head's D channels
      int qe = 0;
      (void)frexpf(qa, &qe);  // qa in [2^(qe - 1), 2^qe)
      const int s = qa > 0.f ? min(10 - qe, 100) : 0;
      const float up = ldexpf(1.f, s);
#pragma unroll
      for (int c = 0; c < E; ++c) {
        const float qt = ((c & 1) ? bf_hi(qw[c >> 1]) : bf_lo(qw[c >> 1])) * up;
        qp[c] = __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)(-int2_off(c) * qt), (_Float16)qt});
      }
      scale2 = p.scale_log2 * ldexpf(1.f, -s);
    }
    // the lane's byte offsets inside a page's head slice, 32-bit so that each load takes the
    // page's address in scalar registers plus one lane offset (lane = 16 g + li)
    const uint32_t off_km = (uint32_t)li * 32u, off_k = 4u * D + (uint32_t)lane * 16u;
    const uint32_t off_vm = (uint32_t)vmeta_off + (uint32_t)(g * 4 + (li >> 2)) * 32u;
    const uint32_t off_lo = 28u * D + (uint32_t)g * 32u + (uint32_t)li * 2u;  // V lo of token g
    constexpr uint32_t kPastSlice = 1u << 30;  // any offset past a slice (plus at most 896)

    // A code page's loads: the head slice of page cp as a buffer resource (live = false: a
    // resource of size 0, whose loads return zeros without touching memory); the key set (K
    // meta of the lane's 8 channels, K codes) and the V set (INT2 V codes, V meta; INT4 V hi
    // goes out with the lo rows in the value phase).
    struct KeyRegs {
      Raw<32> km;
      Raw<16> k0, k1;
    };
    auto far_rsrc = [&](int cp, bool live) {
      return slice_rsrc(p.codes + (uint64_t)tab_code[cp] * p.code_page_bytes + (uint64_t)hk * head_bytes,
                        live ? (uint32_t)head_bytes : 0u);
    };
    auto far_load_k = [&](rsrc_t rs, KeyRegs& kr) {
      buf_load<32, false>(kr.km, rs, off_km);
      buf_load<16, true>(kr.k0, rs, off_k);
      if constexpr (BITS == 4) buf_load<16, true, 1024>(kr.k1, rs, off_k);
    };
    auto far_load_v = [&](rsrc_t rs, Raw<16>& vh, Raw<32>& vm) {
      if constexpr (BITS == 2) buf_load<16, true, (int)(vcode_off - 4 * D)>(vh, rs, off_k);  // INT2 V codes
      buf_load<32, false>(vm, rs, off_vm);
    };
    auto far_load = [&](int cp, rsrc_t& rs, KeyRegs& kr, Raw<16>& vh, Raw<32>& vm) {
      rs = far_rsrc(cp, true);
      far_load_k(rs, kr);
      far_load_v(rs, vh, vm);
    };
    // Key phase of code page cp: K dequant folded into q (LoopKV page, App. E: the
    // per-channel scale multiplies the query, the zero becomes a bias), and the score of
    // the lane's token g + 4 (li / 2) in base-2 units (xs; -inf past the sequence).  A
    // score is bias + sum_c q'_c c_jc over the lane's 8 channels for each of its 8 tokens,
    // then the transposed 16-lane sum.
    auto far_scores = [&](int cp, const KeyRegs& kr, float& xs) {
      const Raw<32>& km = kr.km;
      const Raw<16>& k0 = kr.k0;
      const Raw<16>& k1 = kr.k1;
      // q' = q sigma as one v_fma_mix_f32 with a zero addend (exact in fp32); the codes reach
      // the scores as fp16 pairs (off + c) through v_fma_mix_f32 (the fp16 operand converts
      // exactly), and sum_c off_c q'_c comes off the bias q . z.  INT2: q' from the query
      // pair's fp16 q_c 2^s (2^s too large), and the bias takes one v_dot2 of the pair with
      // the channel's (sigma, z) metadata.
      float qs[E], bias = 0.f;
      if constexpr (BITS == 2) {
#pragma unroll
        for (int c = 0; c < E; ++c) {
          qs[c] = fmaf(f16_hi_f32(qp[c]), f16_to_f32(km.w[c] & 0xFFFFu), 0.f);  // both fp16: exact
          bias = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, qp[c]), __builtin_bit_cast(f16x2_t, km.w[c]),
                                        bias, false);
        }
      } else {
        // INT4: q_c from the bf16 query, one fma per channel for q_c z_c and one for the offset
#pragma unroll
        for (int c = 0; c < E; ++c) {
          const float qc = (c & 1) ? bf_hi(qw[c >> 1]) : bf_lo(qw[c >> 1]);
          qs[c] = fmaf(qc, f16_to_f32(km.w[c] & 0xFFFFu), 0.f);
          bias = fmaf(qc, f16_to_f32(km.w[c] >> 16), bias);
        }
#pragma unroll
        for (int c = 0; c < E; ++c) bias = fmaf(-int4_off(c), qs[c], bias);
      }
      float sc[8];  // slot s: the lane's K code word s, token g + 4 (s ^ (li >> 1)) (kslot)
      if constexpr (BITS == 4) {
        // slots s and 7 - s one after the other: the transposed row sum's first step pairs them,
        // so few scores are held at once
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = (k & 1) ? 7 - (k >> 1) : (k >> 1);
          uint32_t pr[4];
          int4_pairs_f16(i < 4 ? k0.w[i] : k1.w[i - 4], b64, b16, pr);
          float sv = bias;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            sv = fmaf(qs[c], f16_lo_f32(pr[c]), sv);
            sv = fmaf(qs[c + 4], f16_hi_f32(pr[c]), sv);
          }
          sc[i] = sv;
        }
      } else {
        // word j holds slots 2 j and 2 j + 1; each channel's pair feeds both scores
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float sa = bias, sb = bias;
          uint32_t pr[E];
          int2_pairs_f16(k0.w[j], b64, b16, b4, pr);
#pragma unroll
          for (int c = 0; c < E; ++c) {
            sa = fmaf(qs[c], f16_lo_f32(pr[c]), sa);
            sb = fmaf(qs[c], f16_hi_f32(pr[c]), sb);
          }
          sc[2 * j] = sa;
          sc[2 * j + 1] = sb;
        }
      }
      // the row sums of the eight tokens, transposed: this lane keeps the score of its own
      // token g + 4 (li / 2) (base-2 units)
      xs = row_sum16_t8(sc) * scale2;
      // Past the sequence (last page only): score -inf here, and far_head clears those
      // tokens' V meta, so that they get zero weight against finite scales whatever the page
      // holds there.  (Tested as "the last code page": the past-the-end test implies "the
      // page ends past the history", so with that test the compiler dropped the branch and
      // ran it on every page.)
      if (cp == n_cp - 1) {
        if (cp * kCodePage + g + 4 * (li >> 1) >= n_far) xs = -INFINITY;
      }
    };
    auto far_keys = [&](int cp, rsrc_t& rs, float& xs, Raw<16>& vh, Raw<32>& vm) {
      KeyRegs kr;
      far_load(cp, rs, kr, vh, vm);
      far_scores(cp, kr, xs);
    };

    // Value phase, first half: hot test against thr2 (base-2 units), online softmax (the
    // accumulators are rescaled here), the loads of the V lo rows of hot tokens, and the V
    // dequant folded into the weights, which leave as fp16 pairs wpk[j] for tokens 2 j and
    // 2 j + 1 (nearest even); wacc sums the same rounded weights.
    auto far_head = [&](int cp, rsrc_t rs, float xs, float thr2, Raw<32> vm, uint32_t* wpk,
                        uint32_t* lo16, Raw<16>& vh, bool live = true) {
      if (cp == n_cp - 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (cp * kCodePage + g + 4 * i >= n_far) vm.w[i] = 0u;
      }
      // A finite threshold keeps tokens past the sequence (score -inf) cold under any rule,
      // and leaves every finite score hot when the rule's threshold is -inf.
      thr2 = fmaxf(thr2, -3.402823466e38f);  // -FLT_MAX
      const bool hot_own = masked ? xs >= thr2 : xs > -INFINITY;
      // online softmax of this row, one token per lane pair: the page maximum over the row,
      // the lane's own weight, and st.l summing the lane's own weights (the row's sum is
      // half the sum over its lanes).  The reference st.m moves only when the page's maximum
      // passes it, and then to that maximum plus kFarHeadroom, so weights stay at most 1 (the
      // fp16 weight pairs cannot overflow) and a wave skips the rescale of its accumulators
      // on every page where none of its rows passes its reference.
      float mx = dpp_max<0x4E>(xs);  // lanes 2t and 2t + 1 hold the same token
      mx = dpp_max<0x141>(mx);
      mx = dpp_max<0x140>(mx);
      const bool grow = mx > st.m;
      if (lazy_any(grow)) {
        const float mn = grow ? mx + kFarHeadroom : st.m;
        const float alpha = grow ? fast_exp2(st.m - mn) : 1.f;  // 0 from an empty state
        st.l *= alpha;
#pragma unroll
        for (int c = 0; c < E; ++c) o[c] *= alpha;
        zacc *= alpha;
        wacc *= alpha;
        st.m = mn;
      }
      const float mu = (st.m == -INFINITY) ? 0.f : st.m;
      const float p_own = fast_exp2(xs - mu);
      st.l += p_own;
      // every lane needs the eight weights and hot bits: broadcast from lane 2i of the row,
      // the hot bit riding in the sign (a cold or absent token, p = 0 included, has it set)
      const float ps = hot_own ? p_own : -p_own;
      float x[8];
      bool hot[8];
      uint32_t hotbits = 0;
      {
        float pb[8];
        pb[0] = row_bcast<0>(ps);
        pb[1] = row_bcast<2>(ps);
        pb[2] = row_bcast<4>(ps);
        pb[3] = row_bcast<6>(ps);
        pb[4] = row_bcast<8>(ps);
        pb[5] = row_bcast<10>(ps);
        pb[6] = row_bcast<12>(ps);
        pb[7] = row_bcast<14>(ps);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hot[i] = (int32_t)__float_as_uint(pb[i]) >= 0;
          x[i] = fabsf(pb[i]);
          if (TRACE && hot[i]) hotbits |= 1u << (g + 4 * i);
        }
      }
      // V meta of the lane's group for its 8 tokens; fold scale and zero into the weights
      // (tokens past the sequence have p = 0 and cleared meta)
      float wgt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // fma with a zero addend (not a product) so that the f16 operand folds into one
        // v_fma_mix_f32; p sigma >= 0, so the sign of a zero result does not matter
        wgt[i] = fmaf(x[i], f16_to_f32(vm.w[i] & 0xFFFFu), 0.f);  // p sigma
        zacc = fmaf(x[i], f16_to_f32(vm.w[i] >> 16), zacc);        // + p z
        if (masked) zacc = fmaf(1.5f, hot[i] ? 0.f : wgt[i], zacc);  // cold: bucket midpoint
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2_t wp = f16x2_t{(_Float16)wgt[2 * j], (_Float16)wgt[2 * j + 1]};
        wacc = __builtin_amdgcn_fdot2(wp, f16x2_t{(_Float16)1.f, (_Float16)1.f}, wacc, false);
        wpk[j] = __builtin_bit_cast(uint32_t, wp);
      }
      // INT4 and shared cells: the V hi plane goes out with the V lo rows of the hot tokens
      // only (LoopKV page, Sec. 3.3), one memory round trip; the key phase does not need it.
      // A cold token's load takes an offset past the slice, so it returns 0 without a memory
      // access: the loads need no branch, and every wait counts them exactly.
      if constexpr (BITS == 4) buf_load<16, true, (int)(vcode_off - 4 * D)>(vh, rs, off_k);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo16[i] = 0u;
        // token g + 4 i: the token's part of the offset goes in the scalar offset, so that all
        // eight loads share the lane's one offset register
        if constexpr (masked)
          lo16[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, hot[i] ? off_lo : kPastSlice, 128 * i, 0);
      }
      if constexpr (TRACE) {
        const uint32_t word = or4(hotbits);
        if (lane == 0 && live && p.mask_trace) p.mask_trace[((int64_t)b * p.hq + h) * p.mask_words + cp] = word;
      }
    };

    // Value phase, second half: the V codes against the weight pairs, v_dot2c_f32_f16 (the
    // bucket midpoint 1.5 of cold tokens is in zacc, the pairs' offsets come off at the end).
    auto far_tail = [&](const Raw<16>& vh, const uint32_t* lo16, const uint32_t* wpk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2_t wp = __builtin_bit_cast(f16x2_t, wpk[j]);
        if constexpr (BITS == 4) {
          // tokens 2 j and 2 j + 1 (word j of V hi) together: codes 4 hi + lo as fp16 pairs (off
          // + c of token 2 j, off + c of token 2 j + 1) per channel; a cold token's lo is 0.
          // L = lo16[2 j] | lo16[2 j + 1] << 16 as one byte permute of both loads: an op on one
          // conditional load alone would be moved into its branch, with a wait right after the load
          const uint32_t H = vh.w[j], L = __builtin_amdgcn_perm(lo16[2 * j + 1], lo16[2 * j], 0x05040100u);
          uint32_t pr[4];
          int4_pairs_f16(vcodes_lo4(H, L), b64, b16, pr);
#pragma unroll
          for (int c = 0; c < 4; ++c) o[c] = __builtin_amdgcn_fdot2(wp, __builtin_bit_cast(f16x2_t, pr[c]), o[c], false);
          int4_pairs_f16(vcodes_hi4(H, L), b64, b16, pr);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            o[c + 4] = __builtin_amdgcn_fdot2(wp, __builtin_bit_cast(f16x2_t, pr[c]), o[c + 4], false);
        } else {
          // INT2: each channel's pair (off + c of token 2 j, off + c of token 2 j + 1)
          uint32_t pr[E];
          int2_pairs_f16(vh.w[j], b64, b16, b4, pr);
#pragma unroll
          for (int c = 0; c < E; ++c) o[c] = __builtin_amdgcn_fdot2(wp, __builtin_bit_cast(f16x2_t, pr[c]), o[c], false);
        }
      }
    };

    if constexpr (!RUNNING || !masked) {
      // Fixed rule: hot iff s >= m0 - offset.
      const float thr2 = (m0 - p.thr_offset) * kLog2e;
      if constexpr (masked) {
        // INT4 and shared cells: a page's lo rows need its scores, so the wave works on two
        // pages at once.  One step: the scores of page n (its key loads went out one step
        // earlier), the key loads of page n + 1 (into the key registers just freed), the
        // accumulation of page n - 1 (its V hi and lo rows went out one step earlier), the value
        // head of page n (V meta loaded one step earlier; V hi and lo rows go out), and the V
        // meta load of page n + 1.  Every load has a whole phase of other work before its use,
        // each load set reuses the registers of the set it replaces, and after the run's last
        // page the loads go to an empty resource (zeros, no memory access), so no load sits in
        // a branch and every wait counts the loads exactly.
        int cp = c0 + w;
        if (cp < c1) {
          KeyRegs kr;
          Raw<16> vh;
          Raw<32> vm;
          uint32_t wpk[4], lo16[8];
          float xs;
          rsrc_t rs = far_rsrc(cp, true);
          far_load_k(rs, kr);
          far_load_v(rs, vh, vm);
          far_scores(cp, kr, xs);
          int nx = cp + WAVES;
          bool more = nx < c1;
          rsrc_t rs2 = far_rsrc(more ? nx : cp, more);
          far_load_k(rs2, kr);
          far_head(cp, rs, xs, thr2, vm, wpk, lo16, vh);
          far_load_v(rs2, vh, vm);  // (INT4: V meta only; V hi goes out in the head)
          while (more) {
            far_scores(nx, kr, xs);
            const int nn = nx + WAVES;
            const bool more2 = nn < c1;
            const rsrc_t rs3 = far_rsrc(more2 ? nn : nx, more2);
            far_load_k(rs3, kr);
            far_tail(vh, lo16, wpk);
            far_head(nx, rs2, xs, thr2, vm, wpk, lo16, vh);
            far_load_v(rs3, vh, vm);
            nx = nn;
            more = more2;
            rs2 = rs3;
          }
          far_tail(vh, lo16, wpk);
        }
      } else {
        // INT2 cells (no lo rows): the wave issues the next page's key loads as soon as the
        // current page's key registers are free, so they are in flight during its value phase,
        // and the next page's V loads once that phase is done (in flight during the next key
        // phase); each load set reuses the registers of the set it replaces.  After the run's
        // last page the loads go to an empty resource (zeros, no memory access): with no branch
        // around the loads, the waits count them exactly.
        int cp = c0 + w;
        if (cp < c1) {
          rsrc_t rs;
          KeyRegs kr;
          Raw<16> vh;
          Raw<32> vm;
          far_load(cp, rs, kr, vh, vm);
          for (;;) {
            float xs;
            far_scores(cp, kr, xs);
            const int nx = cp + WAVES;
            const bool more = nx < c1;
            const rsrc_t rs2 = far_rsrc(more ? nx : cp, more);
            far_load_k(rs2, kr);
            uint32_t wpk[4], lo16[8];
            far_head(cp, rs, xs, thr2, vm, wpk, lo16, vh);
            far_tail(vh, lo16, wpk);
            far_load_v(rs2, vh, vm);
            if (!more) break;
            cp = nx;
            rs = rs2;
          }
        }
      }
    } else {
      // The LoopKV page's rule (App. E Algorithm 1): this far block walks its pages in order
      // with a running maximum m of its scores so far; a token is hot iff
      // s >= max(m, m0) - tau ln 2, i.e. x2 >= max(m2, m0 log2 e) - tau in base-2 units.
      // The waves take the block's pages in rounds (page c0 + WAVES r + w) and trade page
      // maxima through LDS once per round, so the rule is the sequential one whatever the
      // schedule.  Every wave runs every round, with or without a page, to meet the barrier;
      // a wave without a page in a round (the last one) works on an empty resource with
      // score -inf, which leaves its state unchanged.  The steps overlap as in the fixed-rule
      // loop: a round's key loads go out one round early, its V hi and lo rows are
      // accumulated one round late, and the accumulation of the previous round's page covers
      // the wait at the barrier.
      __shared__ float sm_pm[2][WAVES];
      // m0 and the running maximum are uniform over the wave: kept in scalar registers
      const float m0_2 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(m0 * kLog2e)));
      float m_run = -INFINITY;
      const int n_rounds = (c1 - c0 + WAVES - 1) / WAVES;  // uniform per block
      if (n_rounds > 0) {
        int cp = c0 + w;
        bool live = cp < c1;
        KeyRegs kr;
        Raw<16> vh;
        Raw<32> vm;
        uint32_t wpk[4], lo16[8];
        rsrc_t rs = far_rsrc(live ? cp : c0, live);
        far_load_k(rs, kr);
        far_load_v(rs, vh, vm);
        // One round: the scores of page cp (key loads issued a round earlier), its maximum to
        // LDS, the key loads of the next round's page, the accumulation of the previous round's
        // page (acc), the barrier, the threshold and the value head of page cp (V hi and lo rows
        // go out), and the V meta load of the next round's page.  The first round is its own
        // copy, so that the loop is entered with the loads in flight that its back edge carries.
        auto round_step = [&](int round, bool acc) {
          float xs;
          far_scores(cp, kr, xs);
          if (!live) xs = -INFINITY;
          // the page maximum: over each row (lanes 2t and 2t + 1 hold one token), then the four
          // rows' values read into scalar registers
          float pm = dpp_max<0x4E>(xs);  // -inf past the sequence
          pm = dpp_max<0x141>(pm);
          pm = dpp_max<0x140>(pm);
          const uint32_t pmi = __float_as_uint(pm);
          pm = fmaxf(fmaxf(__uint_as_float(__builtin_amdgcn_readlane(pmi, 0)),
                           __uint_as_float(__builtin_amdgcn_readlane(pmi, 16))),
                     fmaxf(__uint_as_float(__builtin_amdgcn_readlane(pmi, 32)),
                           __uint_as_float(__builtin_amdgcn_readlane(pmi, 48))));
          if (lane == 0) sm_pm[round & 1][w] = pm;
          const int nx = cp + WAVES;
          const bool live2 = nx < c1;
          const rsrc_t rs2 = far_rsrc(live2 ? nx : c0, live2);
          far_load_k(rs2, kr);
          if (acc) far_tail(vh, lo16, wpk);
          __syncthreads();
          float m_page = m_run;
#pragma unroll
          for (int v = 0; v < WAVES; ++v) {
            const float pv = sm_pm[round & 1][v];
            if (v <= w) m_page = fmaxf(m_page, pv);
            m_run = fmaxf(m_run, pv);
          }
          m_run = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(m_run)));
          far_head(cp, rs, xs, fmaxf(m_page, m0_2) - p.v_tau, vm, wpk, lo16, vh, live);
          far_load_v(rs2, vh, vm);
          cp = nx;
          live = live2;
          rs = rs2;
        };
        round_step(0, false);
        for (int round = 1; round < n_rounds; ++round) round_step(round, true);
        far_tail(vh, lo16, wpk);
      }
    }
  }

#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = fmaf(BITS == 4 ? -int4_off(e) : -int2_off(e), wacc, o[e]);  // the pairs' offsets
  st.l = 0.5f * row_sum16(st.l);  // lanes 2t and 2t + 1 hold equal sums, so this is exact

  // merge the block's row states (4 WAVES far rows, and in the near block 4 WAVES near rows)
#pragma unroll
  for (int e = 0; e < E; ++e) sm_o[r][li * E + e] = o[e] + zacc;
  if (li == 0) {
    sm_m[r] = st.m;
    sm_l[r] = st.l;
  }
  __syncthreads();
  const int n_rows = near_block ? WAVES * 8 : WAVES * 4;
  float M = -INFINITY;
  for (int k = 0; k < n_rows; ++k) M = fmaxf(M, sm_m[k]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float Lsum = 0.f;
  for (int k = 0; k < n_rows; ++k) Lsum += sm_l[k] * fast_exp2(sm_m[k] - Mu);
  const int64_t row = (int64_t)b * p.hq + h;
  float* wsr = p.ws + (row * (p.n_splits + 1) + part) * (D + 1);
  for (int c = threadIdx.x; c < D; c += WAVES * 64) {
    float acc = 0.f;
    for (int k = 0; k < n_rows; ++k) acc += sm_o[k][c] * fast_exp2(sm_m[k] - Mu);
    wsr[c] = Lsum > 0.f ? acc / Lsum : 0.f;
  }
  if (threadIdx.x == 0) wsr[D] = Lsum > 0.f ? M + fast_log2(Lsum) : -INFINITY;
}

template <int BITS, bool RUNNING>
static void launch_cell_t(const CellParams& p, int waves, bool trace, dim3 grid, hipStream_t s, const LaunchEvents& ev) {
  if (waves == 2) {
    if (trace) launch_k((cell_kernel<2, true, BITS, RUNNING>), grid, dim3(128), s, ev, p);
    else launch_k((cell_kernel<2, false, BITS, RUNNING>), grid, dim3(128), s, ev, p);
  } else {
    if (trace) launch_k((cell_kernel<4, true, BITS, RUNNING>), grid, dim3(256), s, ev, p);
    else launch_k((cell_kernel<4, false, BITS, RUNNING>), grid, dim3(256), s, ev, p);
  }
}

hipError_t launch_cell(const CellParams& p, int head_dim, int waves, hipStream_t s, const LaunchEvents& ev) {
  if (head_dim != 128 || p.sink < 1 || p.sink > 4 * kPage || (p.bits != 4 && p.bits != 2) || p.masked != (p.bits == 4 ? 1 : 0) ||
      (p.rule != 0 && p.rule != 1))
    return hipErrorInvalidValue;
  dim3 grid(p.n_splits + 1, p.hq, p.n_rows);
  const bool trace = p.mask_trace != nullptr;
  if (p.bits == 2) launch_cell_t<2, false>(p, waves, trace, grid, s, ev);  // INT2 cells have no hot test
  else if (p.rule == 1) launch_cell_t<4, true>(p, waves, trace, grid, s, ev);
  else launch_cell_t<4, false>(p, waves, trace, grid, s, ev);
  return hipGetLastError();
}

}  // namespace lkv
