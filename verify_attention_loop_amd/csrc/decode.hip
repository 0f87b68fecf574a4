// q = 1 attention over plain pages: decode, and the self-speculative draft.
//
// At loop r the query at position t reads, for key j, the plane a policy names
// (RIPE page, Sec. 2 and Eq. (9)): the own plane r for every j under the full
// cache; under RIPE the own plane when t - j <= W or j lies in the query's own
// block, else the deepest plane.  A draft step (RIPE page, Alg. 1) reads cached
// positions through the same rule and its block positions from caller scratch.
//
// Mapping (one workgroup = one (sequence, KV head, split) with its G query heads,
// G = 1 for multi-head attention, 2, 4 or 8 under grouped-query attention; WAVES waves):
//   * a wave takes whole 16-token pages; DPP row g (16 lanes) handles the tokens
//     4i + g of the page, which V quad g holds (page layout in params.hpp);
//   * K: load i of row g reads token 4i + g, lane li its channels
//     [li*E, li*E + E), E = D/16 (dwordx3 for bf16 D = 96), so one load
//     instruction of the wave reads four whole token rows; scores by
//     v_dot2c_f32_bf16 and 16-lane DPP sums;
//   * V: load j of lane li reads 16 B at offset 256 j + 16 li of quad g (two bf16
//     channels or one fp32 channel, four tokens), again whole lines per instruction;
//   * page data is read with nontemporal loads (it is read once per call);
//   * each DPP row keeps its own online softmax (m, l, o); rows and waves merge
//     through LDS at the end, splits through the LSE merge kernel.
// The plane of a key is chosen per token by address, so a RIPE boundary inside a
// page costs one extra V quad load and accumulation pass on that page only.
#include <hip/hip_runtime.h>

#include "attn_common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "params.hpp"

namespace lkv {

// Clears token k of a quad block where zero[k] (slots whose values must not reach the
// sum: they may hold NaN, so they are cleared by select, never by a zero weight).
template <typename T, int D>
__device__ __forceinline__ void clear_quad(Raw<DecodeTile<T, D>::VB>& a, const bool* zero) {
  constexpr int E = D / 16;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int k = 0; k < 4; ++k) a.w[4 * e + k] = zero[k] ? 0u : a.w[4 * e + k];
  } else {
    const uint32_t keep01 = (zero[0] ? 0u : 0x0000FFFFu) | (zero[1] ? 0u : 0xFFFF0000u);
    const uint32_t keep23 = (zero[2] ? 0u : 0x0000FFFFu) | (zero[3] ? 0u : 0xFFFF0000u);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      a.w[2 * e + 0] &= keep01;
      a.w[2 * e + 1] &= keep23;
    }
  }
}

// Seven waves per SIMD fit the multi-head bf16 d = 96 kernel in 66 VGPRs; the hint keeps
// the register allocator there.
template <typename T, int D, int WAVES, bool TRACE, int G>
__global__ __launch_bounds__(WAVES * 64, (G == 1 && D == 96 && sizeof(T) == 2) ? 7 : 1) void decode_kernel(const PlainParams p) {
  using Tl = DecodeTile<T, D>;
  constexpr int E = Tl::E, KB = Tl::KB, VB = Tl::VB, ES = Tl::ES, HEAD = Tl::HEAD;
  // blockIdx.y is the KV head; the workgroup serves its G query heads hk G .. hk G + G - 1
  // (grouped-query attention), so each K/V page is streamed once for all of them.
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int slot = p.slot[b];
  const int n_cached = p.len[b];
  const int L = n_cached + p.draft_len;
  const int t = L - 1;
  const int t0 = p.draft_len > 0 ? n_cached : t;
  const int own_lo = p.ripe ? max(0, min(t0, t - p.window)) : 0;

  // Queries: this lane's channels of each of the G heads.
  float qf[G][E];
  uint32_t qw[G][(E + 1) / 2];
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    const int64_t qbase = ((int64_t)b * p.hq + hk * G + gq) * D + li * E;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int e = 0; e < E; ++e) qf[gq][e] = reinterpret_cast<const float*>(p.q)[qbase + e];
    } else {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + qbase;
#pragma unroll
      for (int e2 = 0; e2 < E / 2; ++e2) qw[gq][e2] = (uint32_t)qp[2 * e2] | ((uint32_t)qp[2 * e2 + 1] << 16);
    }
  }

  const int n_pages = (n_cached + kPage - 1) / kPage;
  const int p0 = (int)((int64_t)split * n_pages / p.n_splits);
  const int p1 = (int)((int64_t)(split + 1) * n_pages / p.n_splits);

  Softmax st[G];
  float o[G][E];
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    st[gq] = Softmax{-INFINITY, 0.f};
#pragma unroll
    for (int e = 0; e < E; ++e) o[gq][e] = 0.f;
  }

  const int32_t* tab_own = p.tab_own + (int64_t)slot * p.ring_own;
  const int32_t* tab_deep = p.tab_deep + (int64_t)slot * p.ring_deep;
  const uint64_t koff = (uint64_t)hk * HEAD + (uint64_t)li * KB;
  const uint64_t voff = (uint64_t)p.hkv * HEAD + (uint64_t)hk * HEAD + (uint64_t)g * (kQuad * D * ES) +
                        (uint64_t)li * 16;

  for (int pg = p0 + w; pg < p1; pg += WAVES) {
    const int pos = pg * kPage;
    // Planes this page is read from: only positions < n_cached count, so a page is
    // never looked up in a plane that none of its valid tokens reads.
    const bool any_own = min(pos + kPage, n_cached) - 1 >= own_lo;
    const bool any_deep = pos < own_lo;
    const int phys_own = any_own ? tab_own[pg % p.ring_own] : 0;
    const int phys_deep = any_deep ? tab_deep[pg] : 0;
    const uint8_t* base_own = p.pool + (uint64_t)phys_own * p.page_bytes;
    const uint8_t* base_deep = p.pool + (uint64_t)phys_deep * p.page_bytes;
    const bool full = pos + kPage <= n_cached;

    Raw<KB> kr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = pos + 4 * i + g;
      const bool own = (j < n_cached) ? (j >= own_lo) : any_own;
      const uint8_t* bp = own ? base_own : base_deep;
      // a lane's K run is one 16-byte piece of a token row: nontemporal when the wave
      // instruction covers whole lines (KB <= 16), plain loads for longer runs
      if constexpr (KB <= 16) load_stream<KB>(kr[i], bp + koff + (uint64_t)(4 * i + g) * (D * ES));
      else load_raw<KB>(kr[i], bp + koff + (uint64_t)(4 * i + g) * (D * ES));
    }
    // A page that straddles the RIPE window edge (rare, wave-uniform) is accumulated in
    // two passes over one V register block: the own plane's tokens first, then the
    // deepest plane's quad loaded into the same registers, so the common path's
    // register budget carries no second quad.
    const bool edge = any_own && any_deep;
    bool take_deep[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) take_deep[k] = edge && pos + 4 * k + g < own_lo;
    Raw<VB> vr;
    load_vquad<T, D>(vr, (any_own ? base_own : base_deep) + voff);
    if (!full || edge) {  // edge or last page: clear the tokens this quad does not supply
      bool zero[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) zero[k] = take_deep[k] || pos + 4 * k + g >= n_cached;
      clear_quad<T, D>(vr, zero);
    }

    float x[G][4];
#pragma unroll
    for (int gq = 0; gq < G; ++gq) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = pos + 4 * i + g;
        const float s = row_sum16(partial_dot<T, D>(kr[i], qf[gq], qw[gq])) * p.scale_log2;
        x[gq][i] = (j < n_cached) ? s : -INFINITY;
      }
      softmax_step<E, 4>(st[gq], o[gq], x[gq]);
      accum_quad<T, D>(o[gq], vr, x[gq]);
    }
    if (edge) {
      load_vquad<T, D>(vr, base_deep + voff);
      bool zero[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) zero[k] = !take_deep[k];
      clear_quad<T, D>(vr, zero);
#pragma unroll
      for (int gq = 0; gq < G; ++gq) accum_quad<T, D>(o[gq], vr, x[gq]);
    }

    if constexpr (TRACE) {
      if (hk == 0 && li == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = pos + 4 * i + g;
          if (j < n_cached && j < p.trace_len) {
            const bool own = j >= own_lo;
            int32_t* tr = p.trace + ((int64_t)b * p.trace_len + j) * 2;
            tr[0] = own ? p.loop : p.deepest;
            tr[1] = (own ? phys_own : phys_deep) * kPage + (j % kPage);
          }
        }
      }
    }
  }

  // Draft block positions from scratch (token-major rows), last split only.
  if (p.draft_len > 0 && split == p.n_splits - 1) {
    for (int i = w * 4 + g; i < p.draft_len; i += WAVES * 4) {
      const int64_t roff = (((int64_t)b * p.draft_len + i) * p.hkv + hk) * D + li * E;
      Raw<KB> kr;
      load_raw<KB>(kr, reinterpret_cast<const uint8_t*>(p.draft_k) + roff * ES);
      // this lane's V channels (vchan) of the draft token
      const uint32_t* vrow = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(p.draft_v) +
                                                               ((((int64_t)b * p.draft_len + i) * p.hkv + hk) * D) * ES);
#pragma unroll
      for (int gq = 0; gq < G; ++gq) {
        float x[1] = {row_sum16(partial_dot<T, D>(kr, qf[gq], qw[gq])) * p.scale_log2};
        softmax_step<E, 1>(st[gq], o[gq], x);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float v;
          if constexpr (sizeof(T) == 4) {
            v = __uint_as_float(vrow[vchan<T>(e, li)]);
          } else {
            const uint32_t pair = vrow[vchan<T>(e & ~1, li) >> 1];
            v = (e & 1) ? bf_hi(pair) : bf_lo(pair);
          }
          o[gq][e] = fmaf(x[0], v, o[gq][e]);
        }
      }
      if constexpr (TRACE) {
        if (hk == 0 && li == 0 && n_cached + i < p.trace_len) {
          int32_t* tr = p.trace + ((int64_t)b * p.trace_len + n_cached + i) * 2;
          tr[0] = p.loop;
          tr[1] = -2;
        }
      }
    }
  }

  // Merge the 4*WAVES row states of this workgroup, one query head at a time.
  __shared__ float sm_o[WAVES * 4][D];
  __shared__ float sm_m[WAVES * 4], sm_l[WAVES * 4];
  const int r = w * 4 + g;
#pragma unroll
  for (int gq = 0; gq < G; ++gq) {
    if (gq > 0) __syncthreads();  // the previous head's reads are done
#pragma unroll
    for (int e = 0; e < E; ++e) sm_o[r][vchan<T>(e, li)] = o[gq][e];
    if (li == 0) {
      sm_m[r] = st[gq].m;
      sm_l[r] = st[gq].l;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < WAVES * 4; ++k) M = fmaxf(M, sm_m[k]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Lsum = 0.f;
#pragma unroll
    for (int k = 0; k < WAVES * 4; ++k) Lsum += sm_l[k] * fast_exp2(sm_m[k] - Mu);
    const int64_t row = (int64_t)b * p.hq + hk * G + gq;
    for (int c = threadIdx.x; c < D; c += WAVES * 64) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < WAVES * 4; ++k) acc += sm_o[k][c] * fast_exp2(sm_m[k] - Mu);
      const float val = Lsum > 0.f ? acc / Lsum : 0.f;
      if (p.n_splits == 1) store_out<T>(p.out, row * D + c, val);
      else p.ws[(row * p.n_splits + split) * (D + 1) + c] = val;
    }
    if (threadIdx.x == 0) {
      const float lse2 = Lsum > 0.f ? M + fast_log2(Lsum) : -INFINITY;
      if (p.n_splits == 1) {
        if (p.lse) p.lse[row] = lse2 * 0.69314718055994531f;
      } else {
        p.ws[(row * p.n_splits + split) * (D + 1) + D] = lse2;
      }
    }
  }
}

// Exact log-sum-exp merge of split partials (LoopKV page, Sec. 3.4): with lse_s the
// base-2 log-sum-exp of part s, o = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M).
// One wave per row; the row's part weights come from one parallel load and a
// butterfly reduction, and the per-channel sums take the parts in index order, so
// the result does not depend on scheduling.  Up to 128 parts.
__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.n_rows) return;  // whole waves leave together
  const int lane = threadIdx.x & 63;
  const float* ws = p.ws + row * p.n_parts * (D + 1);
  const float l0 = lane < p.n_parts ? ws[lane * (D + 1) + D] : -INFINITY;
  const float l1 = lane + 64 < p.n_parts ? ws[(lane + 64) * (D + 1) + D] : -INFINITY;
  const float M = wave_max64(fmaxf(l0, l1));
  const float Mu = (M == -INFINITY) ? 0.f : M;
  const float Ls = wave_sum64(fast_exp2(l0 - Mu) + fast_exp2(l1 - Mu));
  constexpr int NC = (D + 63) / 64;
  float acc[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) acc[k] = 0.f;
#pragma unroll 4
  for (int s = 0; s < p.n_parts; ++s) {
    const float* part = ws + s * (D + 1);
    const float wgt = fast_exp2(part[D] - Mu);  // 0 for an empty part (lse = -inf, o = 0)
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (lane + 64 * k < D) acc[k] = fmaf(wgt, part[lane + 64 * k], acc[k]);
  }
#pragma unroll
  for (int k = 0; k < NC; ++k)
    if (lane + 64 * k < D) store_out<T>(p.out, row * D + lane + 64 * k, Ls > 0.f ? acc[k] / Ls : 0.f);
  if (lane == 0 && p.lse) p.lse[row] = (Ls > 0.f ? M + fast_log2(Ls) : -INFINITY) * 0.69314718055994531f;
}

// ----------------------------------------------------------------------------- launchers

template <typename T, int D, int G>
static void launch_decode_g(const PlainParams& p, int waves, bool trace, hipStream_t s, const LaunchEvents& ev) {
  dim3 grid(p.n_splits, p.hkv, p.n_rows);
  if (waves == 2) {
    if (trace) launch_k((decode_kernel<T, D, 2, true, G>), grid, dim3(128), s, ev, p);
    else launch_k((decode_kernel<T, D, 2, false, G>), grid, dim3(128), s, ev, p);
  } else if (waves == 8) {
    if (trace) launch_k((decode_kernel<T, D, 8, true, G>), grid, dim3(512), s, ev, p);
    else launch_k((decode_kernel<T, D, 8, false, G>), grid, dim3(512), s, ev, p);
  } else {
    if (trace) launch_k((decode_kernel<T, D, 4, true, G>), grid, dim3(256), s, ev, p);
    else launch_k((decode_kernel<T, D, 4, false, G>), grid, dim3(256), s, ev, p);
  }
}

// Group sizes 1 (multi-head), 2, 4 and 8 (grouped-query attention).
template <typename T, int D>
static hipError_t launch_decode_t(const PlainParams& p, int waves, bool trace, hipStream_t s, const LaunchEvents& ev) {
  const int G = p.hq / p.hkv;
  if (G * p.hkv != p.hq) return hipErrorInvalidValue;
  switch (G) {
    case 1: launch_decode_g<T, D, 1>(p, waves, trace, s, ev); break;
    case 2: launch_decode_g<T, D, 2>(p, waves, trace, s, ev); break;
    case 4: launch_decode_g<T, D, 4>(p, waves, trace, s, ev); break;
    case 8: launch_decode_g<T, D, 8>(p, waves, trace, s, ev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const PlainParams& p, int dtype, int head_dim, int waves, bool trace, hipStream_t s, const LaunchEvents& ev) {
  if (dtype == 0) {
    if (head_dim == 64) return launch_decode_t<float, 64>(p, waves, trace, s, ev);
    if (head_dim == 96) return launch_decode_t<float, 96>(p, waves, trace, s, ev);
    if (head_dim == 128) return launch_decode_t<float, 128>(p, waves, trace, s, ev);
  } else {
    if (head_dim == 64) return launch_decode_t<bf16, 64>(p, waves, trace, s, ev);
    if (head_dim == 96) return launch_decode_t<bf16, 96>(p, waves, trace, s, ev);
    if (head_dim == 128) return launch_decode_t<bf16, 128>(p, waves, trace, s, ev);
    if (head_dim == 256) return launch_decode_t<bf16, 256>(p, waves, trace, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, hipStream_t s) {
  if (p.n_parts < 1 || p.n_parts > 128) return hipErrorInvalidValue;
  dim3 grid((p.n_rows + 3) / 4);
  if (dtype == 0) {
    if (head_dim == 64) hipLaunchKernelGGL((merge_kernel<float, 64>), grid, dim3(256), 0, s, p);
    else if (head_dim == 96) hipLaunchKernelGGL((merge_kernel<float, 96>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<float, 128>), grid, dim3(256), 0, s, p);
  } else {
    if (head_dim == 64) hipLaunchKernelGGL((merge_kernel<bf16, 64>), grid, dim3(256), 0, s, p);
    else if (head_dim == 96) hipLaunchKernelGGL((merge_kernel<bf16, 96>), grid, dim3(256), 0, s, p);
    else if (head_dim == 128) hipLaunchKernelGGL((merge_kernel<bf16, 128>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<bf16, 256>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace lkv
