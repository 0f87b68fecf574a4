// q = k verification attention over plain pages (self-speculative verify).
//
// One pass runs a block of k tokens [t0, t0 + k) through loop r; query t reads
// key j <= t from the plane the policy names (RIPE page, Eq. (9); block tokens
// j >= t0 read plane r, proof of Prop. 1).  Under RIPE the rule depends on the
// query, so a page that straddles the window edge is attended twice, once per
// plane, each pass masking the (query, key) pairs the other plane owns.
//
// This is a dense k x 16 x D contraction per page and head, so it runs on MFMA:
//   S^T[16 keys x 16 queries]  = K[16 x D] * Q^T         (16x16x32 bf16 / 16x16x4 f32)
//   O^T[D x 16 queries]       += V^T[D x 16 keys] * P^T   (16x16x16 bf16 / 16x16x4 f32)
// Lane l = (g = l / 16, n = l % 16): n is its query column.  Row m of the K
// operand is the page's token 4 (m % 4) + m / 4, so the lane's S^T values (rows
// 4g..4g+3) are the tokens g, g+4, g+8, g+12 for query n: exactly the P^T operand
// of the PV product, and exactly the four tokens of V quad g, whose
// [channel][4 tokens] layout is the V^T operand (four tokens of one channel per
// lane).  Columns beyond the block are padding.  V is read with nontemporal loads
// (whole lines per instruction); so is K, as the page's contiguous K slice of the KV
// head, staged through LDS, from which each lane reads its operand pieces (16 bytes of
// a token row): read straight from memory those would be 64-byte pieces of 128-512-byte
// rows, partial lines that nontemporal loads serve badly.
//
// Grouped-query attention: with G > 1 a workgroup serves the G query heads of one
// KV head and column c is (block row c / G, head c % G), so every K/V page is read
// once for all G heads.  Blocks of up to 32 such columns (head dim <= 128) take two
// tiles that share the page's K and V registers.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"
#include "params.hpp"

namespace lkv {

// Max and sum over the lanes n, n + 16, n + 32, n + 48 of a query column, on the VALU:
// the gfx950 permlane swaps hand each lane its own value and its partner row's (lanes l
// and l ^ 16, then l and l ^ 32), where a shuffle would go through the LDS crossbar.  Each
// lane adds the same two values as a butterfly would, so sums are unchanged bit for bit.
__device__ __forceinline__ float xmax4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float xsum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <typename T, int D, int WAVES, bool TRACE, int G, int NCT>
__global__ __launch_bounds__(WAVES * 64) void verify_kernel(const PlainParams p) {
  constexpr bool F32 = sizeof(T) == 4;
  constexpr int ES = F32 ? 4 : 2;
  constexpr int HEAD = kPage * D * ES;
  // bf16: D/32 K loads of 8 channels (one 16x16x32 MFMA each) and D/32 V loads of two
  //       channels x 4 tokens (two 16x16x16 MFMAs each).
  // f32:  D/16 K loads of 4 channels (4 MFMAs each); D/16 V loads of one channel x 4 tokens.
  constexpr int NB = F32 ? D / 16 : D / 32;
  constexpr int NACC = F32 ? D / 16 : D / 16;  // 16-channel output blocks
  constexpr int NCOL = 16 * NCT;               // columns of the workgroup's tiles

  // blockIdx.y: the query head (G = 1) or the KV head whose G query heads share the tiles.
  // Column c = 16 t + n (tile t, lane column n) is block row c / G of query head c % G.
  const int split = blockIdx.x, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const int hk = G == 1 ? blockIdx.y / (p.hq / p.hkv) : blockIdx.y;
  const int slot = p.slot[b];
  const int L = p.len[b];
  const int k = p.q_len;
  const int t0 = L - k;
  const int own_min = p.ripe ? max(0, min(t0, t0 - p.window)) : 0;
  const int own_max = p.ripe ? max(0, min(t0, t0 + k - 1 - p.window)) : 0;

  int qi[NCT], h[NCT], tq[NCT], own_n[NCT];
  bool qv[NCT];
  uint32_t qb[NCT][NB][4];  // Q^T operands, zero for padding columns
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
    const int col = 16 * t + n;
    qi[t] = col / G;
    h[t] = blockIdx.y * G + col % G;
    qv[t] = qi[t] < k;
    tq[t] = t0 + qi[t];
    own_n[t] = p.ripe ? max(0, min(t0, tq[t] - p.window)) : 0;
    const int64_t qrow = (((int64_t)b * k + (qv[t] ? qi[t] : 0)) * p.hq + h[t]) * D;
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + qrow * ES;
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      Raw<16> r;
      if constexpr (F32) load_raw<16>(r, qp + (16 * s + 4 * g) * 4);
      else load_raw<16>(r, qp + (32 * s + 8 * g) * 2);
#pragma unroll
      for (int x = 0; x < 4; ++x) qb[t][s][x] = qv[t] ? r.w[x] : 0u;
    }
  }

  f32x4_t acc[NCT][NACC];
  float m[NCT], lsum[NCT];
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[t][a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m[t] = -INFINITY;
    lsum[t] = 0.f;
  }

  const int n_pages = (L + kPage - 1) / kPage;
  const int p0 = (int)((int64_t)split * n_pages / p.n_splits);
  const int p1 = (int)((int64_t)(split + 1) * n_pages / p.n_splits);
  const int32_t* tab_own = p.tab_own + (int64_t)slot * p.ring_own;
  const int32_t* tab_deep = p.tab_deep + (int64_t)slot * p.ring_deep;

  // Per lane: K row token 4 (n % 4) + n / 4 (MFMA row n), channel offsets per load s;
  // V quad g, channels 32 s + 2 n (bf16) or 16 s + n (fp32).
  const uint64_t koff = (uint64_t)hk * HEAD + (uint64_t)(4 * (n & 3) + (n >> 2)) * D * ES +
                        (uint64_t)(F32 ? 4 * g * 4 : 8 * g * 2);
  const uint64_t voff = (uint64_t)p.hkv * HEAD + (uint64_t)hk * HEAD + (uint64_t)g * (kQuad * D * ES) +
                        (uint64_t)(F32 ? n * kQuad * 4 : 2 * n * kQuad * 2);
  constexpr int KSTEP = F32 ? 16 * 4 : 32 * 2;              // bytes between a lane's K loads
  constexpr int VSTEP = F32 ? 16 * kQuad * 4 : 32 * kQuad * 2;  // bytes between a lane's V loads
  // K goes through LDS: the wave reads the page's K slice of its KV head (HEAD bytes,
  // contiguous) with whole-line streaming loads, lane l taking bytes 16 l + 1024 s, and
  // then reads its MFMA operands (row tokens, 16-byte channel pieces) from LDS.
  static_assert(HEAD == NB * 64 * 16, "one 16-byte piece per lane and load");
  __shared__ __attribute__((aligned(16))) uint8_t sm_k[WAVES][HEAD];
  const uint64_t kslice = (uint64_t)hk * HEAD;
  const int kl = (int)(koff - kslice);  // the lane's operand offset inside the slice

  for (int pg = p0 + w; pg < p1; pg += WAVES) {
    const int pos = pg * kPage;
    const int vend = min(pos + kPage, L);
    const bool any_own = vend - 1 >= own_min;  // uniform over the wave; every page has own or deep
    const bool any_deep = pos < own_max;
    for (int pass = any_own ? 0 : 1; pass < (any_deep ? 2 : 1); ++pass) {
      const bool own = pass == 0;
      const int phys = own ? tab_own[pg % p.ring_own] : tab_deep[pg];
      const uint8_t* base = p.pool + (uint64_t)phys * p.page_bytes;
      // Issue every load of the page first: the K slice and the V quads (streaming).
      Raw<16> kr[NB], vr[NB], kst[NB];
#pragma unroll
      for (int s = 0; s < NB; ++s) load_stream<16>(kst[s], base + kslice + (s * 64 + lane) * 16);
#pragma unroll
      for (int s = 0; s < NB; ++s) load_stream<16>(vr[s], base + voff + s * VSTEP);
      // The slice is shared by the lanes of one wave: other lanes' reads of the previous
      // page must be done before it is overwritten, and its stores visible before it is
      // read (wavefront-scope fences around a wave barrier; no workgroup barrier needed).
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int s = 0; s < NB; ++s)
        *reinterpret_cast<u32x4_t*>(&sm_k[w][(s * 64 + lane) * 16]) = u32x4_t{kst[s].w[0], kst[s].w[1], kst[s].w[2], kst[s].w[3]};
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&sm_k[w][kl + s * KSTEP]);
        kr[s].w[0] = v.x;
        kr[s].w[1] = v.y;
        kr[s].w[2] = v.z;
        kr[s].w[3] = v.w;
      }
      // V of tokens this pass does not own is cleared (unused or poisoned slots may hold
      // NaN, and 0 * NaN is NaN); the same for every column
      bool keep[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = pos + 4 * i + g;
        keep[i] = j < L && (own ? j >= own_min : j < own_max);
      }

#pragma unroll
      for (int t = 0; t < NCT; ++t) {
        // ---- S^T = K Q^T
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          if constexpr (F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kr[s].w[e]), __uint_as_float(qb[t][s][e]),
                                                        sc, 0, 0, 0);
          } else {
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[s].w),
                                                         __builtin_bit_cast(bf16x8_t, qb[t][s]), sc, 0, 0, 0);
          }
        }

        // ---- mask, online softmax for the lane's column (S^T element i is token 4i + g)
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = pos + 4 * i + g;
          const bool plane_ok = own ? (j >= own_n[t]) : (j < own_n[t]);
          const bool vis = qv[t] && j <= tq[t] && plane_ok;
          x[i] = vis ? sc[i] * p.scale_log2 : -INFINITY;
          if constexpr (TRACE) {
            if (h[t] == 0 && vis && j < p.trace_len) {  // columns of head 0 only
              int32_t* tr = p.trace + (((int64_t)b * k + qi[t]) * p.trace_len + j) * 2;
              tr[0] = own ? p.loop : p.deepest;
              tr[1] = phys * kPage + (j % kPage);
            }
          }
        }
        // (lazy reference maximum: m moves only when the column's maximum passes it by more
        // than kLazyLog2; from -inf any finite score moves it, with alpha = 0)
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = xmax4(mx);
        const bool grow = mx > m[t] + kLazyLog2;
        const float alpha = grow ? fast_exp2(m[t] - mx) : 1.f;
        if (grow) m[t] = mx;
        const float mu = (m[t] == -INFINITY) ? 0.f : m[t];
        float pe[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pe[i] = fast_exp2(x[i] - mu);
        if (lazy_any(grow)) {
#pragma unroll
          for (int a = 0; a < NACC; ++a) acc[t][a] *= alpha;
        }

        // ---- O^T += V^T P^T
        if constexpr (F32) {
          lsum[t] = fmaf(lsum[t], alpha, (pe[0] + pe[1]) + (pe[2] + pe[3]));
#pragma unroll
          for (int s = 0; s < NB; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float v = __uint_as_float(keep[e] ? vr[s].w[e] : 0u);
              acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, pe[e], acc[t][s], 0, 0, 0);
            }
        } else {
          // P in bf16 for the MFMA; the row sum uses the same rounded weights.
          const uint32_t p01 = pack_bf16x2(pe[0], pe[1]), p23 = pack_bf16x2(pe[2], pe[3]);
          lsum[t] = fmaf(lsum[t], alpha, (bf_lo(p01) + bf_hi(p01)) + (bf_lo(p23) + bf_hi(p23)));
          const uint32_t pw[2] = {p01, p23};
          const uint32_t k01 = (keep[0] ? 0x0000FFFFu : 0u) | (keep[1] ? 0xFFFF0000u : 0u);
          const uint32_t k23 = (keep[2] ? 0x0000FFFFu : 0u) | (keep[3] ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int s = 0; s < NB; ++s) {
            const uint32_t a0[2] = {vr[s].w[0] & k01, vr[s].w[1] & k23};
            const uint32_t a1[2] = {vr[s].w[2] & k01, vr[s].w[3] & k23};
            acc[t][2 * s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(bf16x4_t, a0), __builtin_bit_cast(bf16x4_t, pw), acc[t][2 * s], 0, 0, 0);
            acc[t][2 * s + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(bf16x4_t, a1), __builtin_bit_cast(bf16x4_t, pw), acc[t][2 * s + 1], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- merge the waves of this workgroup through LDS
  __shared__ float sm_o[WAVES][NCOL][D + 1];
  __shared__ float sm_m[WAVES][NCOL], sm_l[WAVES][NCOL];
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
    const float ls = xsum4(lsum[t]);
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int ch;
        if constexpr (F32) ch = 16 * a + 4 * g + i;
        else ch = 32 * (a >> 1) + 2 * (4 * g + i) + (a & 1);
        sm_o[w][16 * t + n][ch] = acc[t][a][i];
      }
    if (g == 0) {
      sm_m[w][16 * t + n] = m[t];
      sm_l[w][16 * t + n] = ls;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < k * G * D; idx += WAVES * 64) {
    const int col = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) M = fmaxf(M, sm_m[v][col]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
      const float f = fast_exp2(sm_m[v][col] - Mu);
      Ls = fmaf(sm_l[v][col], f, Ls);
      O = fmaf(sm_o[v][col][c], f, O);
    }
    const float val = Ls > 0.f ? O / Ls : 0.f;
    const int64_t row = ((int64_t)b * k + col / G) * p.hq + blockIdx.y * G + col % G;
    if (p.n_splits == 1) {
      store_out<T>(p.out, row * D + c, val);
      if (c == 0 && p.lse) p.lse[row] = (Ls > 0.f ? M + fast_log2(Ls) : -INFINITY) * 0.69314718055994531f;
    } else {
      float* wsr = p.ws + (row * p.n_splits + split) * (D + 1);
      wsr[c] = val;
      if (c == 0) wsr[D] = Ls > 0.f ? M + fast_log2(Ls) : -INFINITY;
    }
  }
}

template <typename T, int D, int G, int NCT>
static void launch_verify_g(const PlainParams& p, int waves, bool trace, hipStream_t s, const LaunchEvents& ev) {
  dim3 grid(p.n_splits, p.hq / G, p.n_rows);
  if (waves == 1) {
    if (trace) launch_k((verify_kernel<T, D, 1, true, G, NCT>), grid, dim3(64), s, ev, p);
    else launch_k((verify_kernel<T, D, 1, false, G, NCT>), grid, dim3(64), s, ev, p);
  } else if (waves == 2) {
    if (trace) launch_k((verify_kernel<T, D, 2, true, G, NCT>), grid, dim3(128), s, ev, p);
    else launch_k((verify_kernel<T, D, 2, false, G, NCT>), grid, dim3(128), s, ev, p);
  } else {
    if (trace) launch_k((verify_kernel<T, D, 4, true, G, NCT>), grid, dim3(256), s, ev, p);
    else launch_k((verify_kernel<T, D, 4, false, G, NCT>), grid, dim3(256), s, ev, p);
  }
}

// Query heads per workgroup: the whole group of a KV head when its block rows fit the
// 16 columns of one tile, or (head dim <= 128) two tiles; else one query head.
int verify_heads_per_wg(int hq, int hkv, int q_len, int head_dim) {
  const int group = hq / hkv;
  if (group != 2 && group != 4 && group != 8) return 1;
  return q_len * group <= kMaxBlock || (head_dim <= 128 && q_len * group <= 2 * kMaxBlock) ? group : 1;
}

template <typename T, int D>
static hipError_t launch_verify_t(const PlainParams& p, int waves, bool trace, hipStream_t s, const LaunchEvents& ev) {
  const int G = verify_heads_per_wg(p.hq, p.hkv, p.q_len, D);
  const bool two = p.q_len * G > kMaxBlock;
  if constexpr (D <= 128) {
    if (two) {
      switch (G) {
        case 2: launch_verify_g<T, D, 2, 2>(p, waves, trace, s, ev); return hipGetLastError();
        case 4: launch_verify_g<T, D, 4, 2>(p, waves, trace, s, ev); return hipGetLastError();
        case 8: launch_verify_g<T, D, 8, 2>(p, waves, trace, s, ev); return hipGetLastError();
        default: return hipErrorInvalidValue;
      }
    }
  }
  switch (G) {
    case 2: launch_verify_g<T, D, 2, 1>(p, waves, trace, s, ev); break;
    case 4: launch_verify_g<T, D, 4, 1>(p, waves, trace, s, ev); break;
    case 8: launch_verify_g<T, D, 8, 1>(p, waves, trace, s, ev); break;
    default: launch_verify_g<T, D, 1, 1>(p, waves, trace, s, ev); break;
  }
  return hipGetLastError();
}

hipError_t launch_verify(const PlainParams& p, int dtype, int head_dim, int waves, bool trace, hipStream_t s, const LaunchEvents& ev) {
  if (p.q_len < 1 || p.q_len > kMaxBlock || p.draft_len != 0) return hipErrorInvalidValue;
  if (p.hkv < 1 || p.hq % p.hkv != 0) return hipErrorInvalidValue;
  if (waves != 1 && waves != 2) waves = 4;
  if (dtype == 0) {
    if (head_dim == 64) return launch_verify_t<float, 64>(p, waves, trace, s, ev);
    if (head_dim == 96) return launch_verify_t<float, 96>(p, waves, trace, s, ev);
    if (head_dim == 128) return launch_verify_t<float, 128>(p, waves, trace, s, ev);
  } else {
    if (head_dim == 64) return launch_verify_t<bf16, 64>(p, waves, trace, s, ev);
    if (head_dim == 96) return launch_verify_t<bf16, 96>(p, waves, trace, s, ev);
    if (head_dim == 128) return launch_verify_t<bf16, 128>(p, waves, trace, s, ev);
    if (head_dim == 256) return launch_verify_t<bf16, 256>(p, waves, trace, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace lkv
