// q = 1 decode of a grouped-query cache on MFMA.
//
// Query head h reads KV head h / G (grouped-query attention, as in the Raven and
// Dory models of the LoopKV page).  One workgroup = one (sequence, KV head, split);
// its G query heads are G columns of one 16-column MFMA tile, so each K/V page is
// streamed once for all of them and the softmax work per page does not grow with G:
//   S^T[16 keys x 16 cols]  = K[16 x D] * Q^T         (16x16x32 bf16 / 16x16x4 f32)
//   O^T[D x 16 cols]       += V^T[D x 16 keys] * P^T   (16x16x16 bf16 / 16x16x4 f32)
// Row m of the K operand is the page's token 4 (m % 4) + m / 4, so lane (g, n) holds
// the scores of tokens g, g + 4, g + 8, g + 12 for column n: the P^T operand of the
// PV product and the four tokens of V quad g, whose [channel][4 tokens] layout is
// the V^T operand.  Columns G..15 are padding.
//
// Plane of key j for the query at t = L - 1 (RIPE page, Eq. (9)): the own plane when
// t - j <= W (every key under the full cache), else the deepest plane.  The choice is
// the same for all G columns, so it is made per token by address: K rows load from
// their plane, and a page that straddles the window edge loads both V quads and
// blends them per token.
//
// Each wave walks its pages with two register buffers (d <= 128): the loads of its
// next page are in flight while it computes the current one.  V is read with nontemporal
// loads (whole lines per instruction); K rows are 64-byte pieces of 128-256-byte
// token rows, so they use plain loads, which L2 merges.
#include <hip/hip_runtime.h>

#include "attn_common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "params.hpp"

namespace lkv {

namespace {

// Max and sum over the lanes n, n + 16, n + 32, n + 48 of a column, on the VALU: the
// gfx950 permlane swaps hand each lane its own value and its partner row's (lanes l and
// l ^ 16, then l and l ^ 32), where a shuffle would go through the LDS crossbar.  Each
// lane adds the same two values as a butterfly would, so sums are unchanged bit for bit.
__device__ __forceinline__ float col_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float col_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One page's operands in registers: K rows of the lane's token, V quad block.
template <typename T, int D>
struct PageRegs {
  static constexpr int NB = sizeof(T) == 4 ? D / 16 : D / 32;
  Raw<16> k[NB];
  Raw<DecodeTile<T, D>::VB> v;
  int phys_own, phys_deep;
  bool own_tok;  // plane of the lane's K row token (for the trace)
  bool edge;     // the page straddles the RIPE window edge (uniform over the wave)
};

}  // namespace

template <typename T, int D, int WAVES, bool TRACE, int G>
__global__ __launch_bounds__(WAVES * 64, D == 256 ? 2 : 1) void gqa_decode_kernel(const PlainParams p) {
  using Tl = DecodeTile<T, D>;
  using PR = PageRegs<T, D>;
  constexpr bool F32 = sizeof(T) == 4;
  constexpr int ES = Tl::ES, HEAD = Tl::HEAD, NB = PR::NB;
  constexpr int NACC = D / 16;  // 16-channel output blocks

  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const bool qv = n < G;
  const int slot = p.slot[b];
  const int L = p.len[b];
  const int own_lo = p.ripe ? max(0, L - 1 - p.window) : 0;

  // Q^T operand: column n is query head hk G + n; padding columns are zero.
  uint32_t qb[NB][4];
  {
    const int64_t qrow = ((int64_t)b * p.hq + hk * G + (qv ? n : 0)) * D;
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + qrow * ES;
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      Raw<16> r;
      load_raw<16>(r, qp + (F32 ? (16 * s + 4 * g) * 4 : (32 * s + 8 * g) * 2));
#pragma unroll
      for (int x = 0; x < 4; ++x) qb[s][x] = qv ? r.w[x] : 0u;
    }
  }

  f32x4_t acc[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  const int n_pages = (L + kPage - 1) / kPage;
  const int p0 = (int)((int64_t)split * n_pages / p.n_splits);
  const int p1 = (int)((int64_t)(split + 1) * n_pages / p.n_splits);
  const int32_t* tab_own = p.tab_own + (int64_t)slot * p.ring_own;
  const int32_t* tab_deep = p.tab_deep + (int64_t)slot * p.ring_deep;
  const int krow = 4 * (n & 3) + (n >> 2);  // token of the lane's K operand row
  const uint64_t koff = (uint64_t)hk * HEAD + (uint64_t)krow * D * ES + 16 * g;
  const uint64_t voff = (uint64_t)p.hkv * HEAD + (uint64_t)hk * HEAD + (uint64_t)g * (kQuad * D * ES) + 16 * n;

  // K goes through LDS on a page of one plane (every page but the one at the RIPE window
  // edge): the wave reads the page's K slice of its KV head (HEAD bytes, contiguous) with
  // whole-line streaming loads, lane l taking bytes 16 l + 1024 s, and then reads its MFMA
  // operand pieces (row krow, 16-byte channel pieces 64 bytes apart) from LDS.  On the edge
  // page each lane reads its operand pieces straight from its token's plane.
  static_assert(HEAD == NB * 64 * 16, "one 16-byte piece per lane and load");
  __shared__ __attribute__((aligned(16))) uint8_t sm_k[WAVES][HEAD];
  const int kl = (int)(koff - (uint64_t)hk * HEAD);  // the lane's operand offset inside the slice

  // Issue the loads of page pg (no waits: the page's per-token plane choice for V waits
  // until compute_page).
  auto load_page = [&](int pg, PR& r) {
    const int pos = pg * kPage;
    const bool any_own = min(pos + kPage, L) - 1 >= own_lo;
    const bool any_deep = pos < own_lo;
    r.phys_own = any_own ? tab_own[pg % p.ring_own] : 0;
    r.phys_deep = any_deep ? tab_deep[pg] : 0;
    const uint8_t* base_own = p.pool + (uint64_t)r.phys_own * p.page_bytes;
    const uint8_t* base_deep = p.pool + (uint64_t)r.phys_deep * p.page_bytes;
    const int jk = pos + krow;
    r.own_tok = jk < L ? jk >= own_lo : any_own;
    r.edge = any_own && any_deep;
    const uint8_t* kb = (r.own_tok ? base_own : base_deep) + koff;                                    // edge page
    const uint8_t* ks = (any_own ? base_own : base_deep) + (uint64_t)hk * HEAD + (uint64_t)lane * 16;  // slice
#pragma unroll
    for (int s = 0; s < NB; ++s) load_stream<16>(r.k[s], r.edge ? kb + 64 * s : ks + 1024 * s);
    load_vquad<T, D>(r.v, (any_own ? base_own : base_deep) + voff);
  };

  // Scores, online softmax and weighted sum of one loaded page.
  auto compute_page = [&](int pg, const PR& r) {
    const int pos = pg * kPage;
    // V: at the last page and the window edge the plane is chosen per token (the edge's
    // plane-R quad is loaded here, once, since the case is rare) and tokens past the
    // sequence are cleared
    Raw<Tl::VB> v = r.v;
    {
      const bool any_own = min(pos + kPage, L) - 1 >= own_lo;
      const bool any_deep = pos < own_lo;
      if (pos + kPage > L || (any_own && any_deep)) {  // last page or window edge: per-token plane, validity
        Raw<Tl::VB> vd;
        if (any_own && any_deep) load_vquad<T, D>(vd, p.pool + (uint64_t)r.phys_deep * p.page_bytes + voff);
        bool take_deep[4], zero[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = pos + 4 * i + g;
          take_deep[i] = any_own && any_deep && j < own_lo;
          zero[i] = j >= L;
        }
        blend_quad<T, D>(v, vd, take_deep, zero);
      }
    }
    // the K operand: staged through the wave's LDS slice, or (edge page) as loaded
    Raw<16> kop[NB];
#pragma unroll
    for (int s = 0; s < NB; ++s) kop[s] = r.k[s];
    if (!r.edge) {
      // the slice is shared by the lanes of one wave: other lanes' reads of the previous
      // page must be done before it is overwritten, and its stores visible before it is
      // read (wavefront-scope fences around a wave barrier)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int s = 0; s < NB; ++s)
        *reinterpret_cast<u32x4_t*>(&sm_k[w][(s * 64 + lane) * 16]) = u32x4_t{r.k[s].w[0], r.k[s].w[1], r.k[s].w[2], r.k[s].w[3]};
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        const u32x4_t v4 = *reinterpret_cast<const u32x4_t*>(&sm_k[w][kl + 64 * s]);
        kop[s].w[0] = v4.x;
        kop[s].w[1] = v4.y;
        kop[s].w[2] = v4.z;
        kop[s].w[3] = v4.w;
      }
    }
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kop[s].w[e]), __uint_as_float(qb[s][e]), sc, 0,
                                                    0, 0);
      } else {
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[s].w),
                                                     __builtin_bit_cast(bf16x8_t, qb[s]), sc, 0, 0, 0);
      }
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = pos + 4 * i + g < L ? sc[i] * p.scale_log2 : -INFINITY;
    // lazy reference maximum (m moves only when the column's maximum passes it by more than
    // kLazyLog2; from -inf any finite score moves it, with alpha = 0)
    const float mx = col_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const bool grow = mx > m + kLazyLog2;
    const float alpha = grow ? fast_exp2(m - mx) : 1.f;
    if (grow) m = mx;
    const float mu = (m == -INFINITY) ? 0.f : m;
    float pe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pe[i] = fast_exp2(x[i] - mu);
    if (lazy_any(grow)) {
#pragma unroll
      for (int a = 0; a < NACC; ++a) acc[a] *= alpha;
    }
    if constexpr (F32) {
      lsum = fmaf(lsum, alpha, (pe[0] + pe[1]) + (pe[2] + pe[3]));
#pragma unroll
      for (int s = 0; s < NACC; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.w[4 * s + e]), pe[e], acc[s], 0, 0, 0);
    } else {
      // P in bf16 for the MFMA; the row sum uses the same rounded weights.
      const uint32_t p01 = pack_bf16x2(pe[0], pe[1]), p23 = pack_bf16x2(pe[2], pe[3]);
      lsum = fmaf(lsum, alpha, (bf_lo(p01) + bf_hi(p01)) + (bf_lo(p23) + bf_hi(p23)));
      const uint32_t pw[2] = {p01, p23};
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        const uint32_t vw[2] = {v.w[2 * a], v.w[2 * a + 1]};
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, vw),
                                                           __builtin_bit_cast(bf16x4_t, pw), acc[a], 0, 0, 0);
      }
    }
    if constexpr (TRACE) {
      if (hk == 0 && g == 0) {  // lane n of the first row holds K row krow of the page
        const int j = pos + krow;
        if (j < L && j < p.trace_len) {
          int32_t* tr = p.trace + ((int64_t)b * p.trace_len + j) * 2;
          tr[0] = r.own_tok ? p.loop : p.deepest;
          tr[1] = (r.own_tok ? r.phys_own : r.phys_deep) * kPage + (j % kPage);
        }
      }
    }
  };

  // The wave's pages are p0 + w, p0 + w + WAVES, ...  Up to d = 128 two register buffers
  // (a: even pages, b: odd) keep the next page's loads in flight; at d = 256 one page's
  // operands are 64 VGPRs, and a single buffer keeps two waves per SIMD.  No prefetch
  // sits inside a branch that rejoins before the compute it overlaps (the run's last
  // page leaves the loop instead): the compiler's wait before a page then counts only
  // the loads issued before it, where a conditional prefetch made it wait for all.
  if constexpr (D <= 128) {
    int pa = p0 + w;
    if (pa < p1) {
      PR ra, rb;
      load_page(pa, ra);
      while (true) {
        const int pb = pa + WAVES;
        if (pb >= p1) {
          compute_page(pa, ra);
          break;
        }
        load_page(pb, rb);
        compute_page(pa, ra);
        const int pc = pb + WAVES;
        if (pc >= p1) {
          compute_page(pb, rb);
          break;
        }
        load_page(pc, ra);
        compute_page(pb, rb);
        pa = pc;
      }
    }
  } else {
    for (int pa = p0 + w; pa < p1; pa += WAVES) {
      PR ra;
      load_page(pa, ra);
      compute_page(pa, ra);
    }
  }
  lsum = col_sum(lsum);

  // Merge the waves of this workgroup through LDS (columns 0..G-1).
  __shared__ float sm_o[WAVES][G][D + 1];
  __shared__ float sm_m[WAVES][G], sm_l[WAVES][G];
  if (qv) {
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // O^T block a, row 4 g + i: V element 4 g + i of load a / 2 (bf16) or channel 16 a + 4 g + i (fp32)
        const int ch = F32 ? 16 * a + 4 * g + i : 32 * (a >> 1) + 2 * (4 * g + i) + (a & 1);
        sm_o[w][n][ch] = acc[a][i];
      }
    if (g == 0) {
      sm_m[w][n] = m;
      sm_l[w][n] = lsum;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += WAVES * 64) {
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
    const int64_t row = (int64_t)b * p.hq + hk * G + col;
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

template <typename T, int D, int G>
static void launch_gqa_g(const PlainParams& p, int waves, bool trace, hipStream_t s, const LaunchEvents& ev) {
  dim3 grid(p.n_splits, p.hkv, p.n_rows);
  if (waves == 1) {
    if (trace) launch_k((gqa_decode_kernel<T, D, 1, true, G>), grid, dim3(64), s, ev, p);
    else launch_k((gqa_decode_kernel<T, D, 1, false, G>), grid, dim3(64), s, ev, p);
  } else if (waves == 2) {
    if (trace) launch_k((gqa_decode_kernel<T, D, 2, true, G>), grid, dim3(128), s, ev, p);
    else launch_k((gqa_decode_kernel<T, D, 2, false, G>), grid, dim3(128), s, ev, p);
  } else {
    if (trace) launch_k((gqa_decode_kernel<T, D, 4, true, G>), grid, dim3(256), s, ev, p);
    else launch_k((gqa_decode_kernel<T, D, 4, false, G>), grid, dim3(256), s, ev, p);
  }
}

template <typename T, int D>
static hipError_t launch_gqa_t(const PlainParams& p, int waves, bool trace, hipStream_t s, const LaunchEvents& ev) {
  switch (p.hq / p.hkv) {
    case 2: launch_gqa_g<T, D, 2>(p, waves, trace, s, ev); break;
    case 4: launch_gqa_g<T, D, 4>(p, waves, trace, s, ev); break;
    case 8: launch_gqa_g<T, D, 8>(p, waves, trace, s, ev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Grouped-query decode (group 2, 4 or 8; q = 1, no draft block).
hipError_t launch_gqa_decode(const PlainParams& p, int dtype, int head_dim, int waves, bool trace, hipStream_t s, const LaunchEvents& ev) {
  if (p.q_len != 1 || p.draft_len != 0 || p.hkv < 1 || p.hq % p.hkv != 0) return hipErrorInvalidValue;
  if (waves != 1 && waves != 2) waves = 4;
  if (dtype == 0) {
    if (head_dim == 64) return launch_gqa_t<float, 64>(p, waves, trace, s, ev);
    if (head_dim == 96) return launch_gqa_t<float, 96>(p, waves, trace, s, ev);
    if (head_dim == 128) return launch_gqa_t<float, 128>(p, waves, trace, s, ev);
  } else {
    if (head_dim == 64) return launch_gqa_t<bf16, 64>(p, waves, trace, s, ev);
    if (head_dim == 96) return launch_gqa_t<bf16, 96>(p, waves, trace, s, ev);
    if (head_dim == 128) return launch_gqa_t<bf16, 128>(p, waves, trace, s, ev);
    if (head_dim == 256) return launch_gqa_t<bf16, 256>(p, waves, trace, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace lkv
