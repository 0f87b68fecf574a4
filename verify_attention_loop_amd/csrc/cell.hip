// LoopKV-style quantised cells: packed code pages and the cell attention kernel.
//
// Code page (32 far-history tokens of one (seq, layer, loop) cell, all KV heads;
// head_dim 128).  Per head, INT4 (40 * D bytes = 160 B per token-head: 4-bit K and
// V codes plus fp16 scale/zero per 32 elements, LoopKV page App. C):
//   [0,    4D)  K meta   [channel][scale, zero] fp16, per channel over the page
//   [4D,  20D)  K codes  4-bit, lane-major: [half][g][li][4 tokens][8 nibbles]
//   [20D, 28D)  V hi     2-bit hi = c >> 2, lane-major: [g][li][8 tokens][8 x 2 bits]
//   [28D, 36D)  V lo     2-bit lo = c & 3, token-major: [token][D x 2 bits]
//   [36D, 40D)  V meta   [g][group][8 tokens][scale, zero] fp16, per token and 32 channels
// INT2 (24 * D bytes): K meta [0,4D), K codes [4D,12D) as V hi, V codes [12D,20D)
// as V hi, V meta [20D,24D).  Lane (g, li) of a DPP row owns channels 8li..8li+7
// and tokens g, g+4, ..., g+28 of the page, so its K codes, V hi and V meta are
// contiguous 16-32 B runs; V lo is token-major so that a cold token's 32-byte lo
// row (one token-head) is never requested at all (LoopKV page, Sec. 3.3).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "params.hpp"

namespace lkv {

uint64_t code_page_bytes(int hkv, int head_dim, int bits) {
  return (uint64_t)hkv * (bits == 4 ? 40 : 24) * head_dim;
}

// One thread per (head, token, lane li): packs that lane's 8 channels of one token.
__global__ __launch_bounds__(256) void pack_codes_kernel(uint8_t* page, const uint8_t* kc, const uint16_t* km,
                                                         const uint8_t* vc, const uint16_t* vm, int hkv, int bits) {
  constexpr int D = 128;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= hkv * kCodePage * 16) return;
  const int li = idx & 15;
  const int tok = (idx >> 4) & 31;
  const int h = idx >> 9;
  const int g = tok & 3, i = tok >> 2;
  uint8_t* hb = page + (uint64_t)h * (bits == 4 ? 40 : 24) * D;
  const uint8_t* kin = kc + ((int64_t)tok * hkv + h) * D + 8 * li;
  const uint8_t* vin = vc + ((int64_t)tok * hkv + h) * D + 8 * li;
  if (bits == 4) {
    uint32_t kw = 0, vhi = 0, vlo = 0;
    for (int c = 0; c < 8; ++c) {
      kw |= (uint32_t)(kin[c] & 15u) << (4 * c);
      vhi |= (uint32_t)((vin[c] >> 2) & 3u) << (2 * c);
      vlo |= (uint32_t)(vin[c] & 3u) << (2 * c);
    }
    const int hh = i >> 2, ii = i & 3;
    *reinterpret_cast<uint32_t*>(hb + 4 * D + hh * 1024 + (g * 16 + li) * 16 + ii * 4) = kw;
    *reinterpret_cast<uint16_t*>(hb + 20 * D + (g * 16 + li) * 16 + i * 2) = (uint16_t)vhi;
    *reinterpret_cast<uint16_t*>(hb + 28 * D + tok * 32 + li * 2) = (uint16_t)vlo;
  } else {
    uint32_t kw = 0, vw = 0;
    for (int c = 0; c < 8; ++c) {
      kw |= (uint32_t)(kin[c] & 3u) << (2 * c);
      vw |= (uint32_t)(vin[c] & 3u) << (2 * c);
    }
    *reinterpret_cast<uint16_t*>(hb + 4 * D + (g * 16 + li) * 16 + i * 2) = (uint16_t)kw;
    *reinterpret_cast<uint16_t*>(hb + 12 * D + (g * 16 + li) * 16 + i * 2) = (uint16_t)vw;
  }
  // V meta: group li & 3 of this token (threads li < 4)
  if (li < 4) {
    const int grp = li;
    const uint16_t* src = vm + (((int64_t)tok * hkv + h) * (D / 32) + grp) * 2;
    uint16_t* dst = reinterpret_cast<uint16_t*>(hb + (bits == 4 ? 36 : 20) * D + ((g * 4 + grp) * 8 + i) * 4);
    dst[0] = src[0];
    dst[1] = src[1];
  }
  // K meta: channel tok * 16 + li (tokens 0..7 cover the 128 channels)
  if (tok < 8) {
    const int c = tok * 16 + li;
    const uint16_t* src = km + ((int64_t)h * D + c) * 2;
    uint16_t* dst = reinterpret_cast<uint16_t*>(hb + c * 4);
    dst[0] = src[0];
    dst[1] = src[1];
  }
}

hipError_t launch_pack_codes(uint8_t* page, const void* k_codes, const void* k_meta, const void* v_codes,
                             const void* v_meta, int hkv, int head_dim, int bits, int n_valid, hipStream_t s) {
  (void)n_valid;
  if (head_dim != 128) return hipErrorInvalidValue;
  const int n = hkv * kCodePage * 16;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((n + 255) / 256), dim3(256), 0, s, page,
                     reinterpret_cast<const uint8_t*>(k_codes), reinterpret_cast<const uint16_t*>(k_meta),
                     reinterpret_cast<const uint8_t*>(v_codes), reinterpret_cast<const uint16_t*>(v_meta), hkv, bits);
  return hipGetLastError();
}

hipError_t launch_cell(const CellParams& p, int head_dim, int waves, hipStream_t s) {
  (void)p;
  (void)head_dim;
  (void)waves;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace lkv
