// q = 1 attention over plain pages: decode, and the self-speculative draft.
//
// At loop r the query at position t reads, for key j, the plane a policy names
// (RIPE page, Sec. 2 and Eq. (9)): the own plane r for every j under the full
// cache; under RIPE the own plane when t - j <= W or j lies in the query's own
// block, else the deepest plane.  A draft step (RIPE page, Alg. 1) reads cached
// positions through the same rule and its block positions from caller scratch.
//
// Mapping (one workgroup = one (sequence, query head, split) row, WAVES waves):
//   * a wave takes whole 16-token pages; its 4 DPP rows of 16 lanes take the
//     page's 4 quads, lane li owning channels [li*E, li*E + E), E = D/16;
//   * K: row g reads token 4g+i of the page per load i (E*2 bytes per lane,
//     dwordx3 for D = 96), dot products by v_dot2c_f32_bf16, 16-lane DPP sums;
//   * V: row g reads its quad's [channel][4 tokens] block, 16 B per lane-load;
//   * each DPP row keeps its own online softmax (m, l, o); rows and waves merge
//     through LDS at the end, splits through the LSE merge kernel.
// The plane of a key is chosen per token by address, so a RIPE boundary inside a
// page costs one extra V quad load on that page only.
#include <hip/hip_runtime.h>

#include "attn_common.hpp"
#include "device.hpp"
#include "params.hpp"

namespace lkv {

template <typename T, int D, int WAVES, bool TRACE>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(const PlainParams p) {
  using Tl = DecodeTile<T, D>;
  constexpr int E = Tl::E, KB = Tl::KB, VB = Tl::VB, ES = Tl::ES, HEAD = Tl::HEAD;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int hk = h / (p.hq / p.hkv);
  const int slot = p.slot[b];
  const int n_cached = p.len[b];
  const int L = n_cached + p.draft_len;
  const int t = L - 1;
  const int t0 = p.draft_len > 0 ? n_cached : t;
  const int own_lo = p.ripe ? max(0, min(t0, t - p.window)) : 0;

  // Query: this lane's channels.
  float qf[E];
  uint32_t qw[(E + 1) / 2];
  {
    const int64_t qbase = ((int64_t)b * p.hq + h) * D + li * E;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int e = 0; e < E; ++e) qf[e] = reinterpret_cast<const float*>(p.q)[qbase + e];
    } else {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + qbase;
#pragma unroll
      for (int e2 = 0; e2 < E / 2; ++e2) qw[e2] = (uint32_t)qp[2 * e2] | ((uint32_t)qp[2 * e2 + 1] << 16);
    }
  }

  const int n_pages = (n_cached + kPage - 1) / kPage;
  const int p0 = (int)((int64_t)split * n_pages / p.n_splits);
  const int p1 = (int)((int64_t)(split + 1) * n_pages / p.n_splits);

  Softmax st{-INFINITY, 0.f};
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;

  const int32_t* tab_own = p.tab_own + (int64_t)slot * p.ring_own;
  const int32_t* tab_deep = p.tab_deep + (int64_t)slot * p.ring_deep;
  const uint64_t koff = (uint64_t)hk * HEAD + (uint64_t)li * KB;
  const uint64_t voff = (uint64_t)p.hkv * HEAD + (uint64_t)hk * HEAD + (uint64_t)g * (kQuad * D * ES) +
                        (uint64_t)li * VB;

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
      const int j = pos + 4 * g + i;
      const bool own = (j < n_cached) ? (j >= own_lo) : any_own;
      const uint8_t* bp = own ? base_own : base_deep;
      load_raw<KB>(kr[i], bp + koff + (uint64_t)(4 * g + i) * (D * ES));
    }
    Raw<VB> vr;
    load_raw<VB>(vr, (any_own ? base_own : base_deep) + voff);
    if (!full || (any_own && any_deep)) {  // boundary or last page: per-token plane and validity
      Raw<VB> vd;
      if (any_own && any_deep) load_raw<VB>(vd, base_deep + voff);
      bool take_deep[4], zero[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = pos + 4 * g + k;
        take_deep[k] = any_own && any_deep && j < own_lo;
        zero[k] = j >= n_cached;
      }
      blend_quad<T, D>(vr, vd, take_deep, zero);
    }

    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = pos + 4 * g + i;
      const float s = row_sum16(partial_dot<T, D>(kr[i], qf, qw)) * p.scale_log2;
      x[i] = (j < n_cached) ? s : -INFINITY;
    }
    softmax_step<E, 4>(st, o, x);
    accum_quad<T, D>(o, vr, x);

    if constexpr (TRACE) {
      if (h == 0 && li == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = pos + 4 * g + i;
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
      Raw<KB> vr;
      load_raw<KB>(kr, reinterpret_cast<const uint8_t*>(p.draft_k) + roff * ES);
      load_raw<KB>(vr, reinterpret_cast<const uint8_t*>(p.draft_v) + roff * ES);
      float x[1] = {row_sum16(partial_dot<T, D>(kr, qf, qw)) * p.scale_log2};
      softmax_step<E, 1>(st, o, x);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float v;
        if constexpr (sizeof(T) == 4) v = __uint_as_float(vr.w[e]);
        else v = (e & 1) ? bf_hi(vr.w[e >> 1]) : bf_lo(vr.w[e >> 1]);
        o[e] = fmaf(x[0], v, o[e]);
      }
      if constexpr (TRACE) {
        if (h == 0 && li == 0 && n_cached + i < p.trace_len) {
          int32_t* tr = p.trace + ((int64_t)b * p.trace_len + n_cached + i) * 2;
          tr[0] = p.loop;
          tr[1] = -2;
        }
      }
    }
  }

  // Merge the 4*WAVES row states of this workgroup.
  __shared__ float sm_o[WAVES * 4][D];
  __shared__ float sm_m[WAVES * 4], sm_l[WAVES * 4];
  const int r = w * 4 + g;
#pragma unroll
  for (int e = 0; e < E; ++e) sm_o[r][li * E + e] = o[e];
  if (li == 0) {
    sm_m[r] = st.m;
    sm_l[r] = st.l;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < WAVES * 4; ++k) M = fmaxf(M, sm_m[k]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float Lsum = 0.f;
#pragma unroll
  for (int k = 0; k < WAVES * 4; ++k) Lsum += sm_l[k] * fast_exp2(sm_m[k] - Mu);
  const int64_t row = (int64_t)b * p.hq + h;
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

// Exact log-sum-exp merge of split partials (LoopKV page, Sec. 3.4): with
// lse_s the base-2 log-sum-exp of split s, o = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M).
template <typename T, int D>
__global__ __launch_bounds__(128) void merge_kernel(const MergeParams p) {
  const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 6);
  if (row >= p.n_rows) return;
  const int lane = threadIdx.x & 63;
  const float* ws = p.ws + row * p.n_parts * (D + 1);
  float M = -INFINITY;
  for (int s = 0; s < p.n_parts; ++s) M = fmaxf(M, ws[s * (D + 1) + D]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float Ls = 0.f;
  for (int s = 0; s < p.n_parts; ++s) Ls += fast_exp2(ws[s * (D + 1) + D] - Mu);
  for (int c = lane; c < D; c += 64) {
    float acc = 0.f;
    for (int s = 0; s < p.n_parts; ++s) {
      const float wgt = fast_exp2(ws[s * (D + 1) + D] - Mu);
      if (wgt > 0.f) acc = fmaf(wgt, ws[s * (D + 1) + c], acc);
    }
    store_out<T>(p.out, row * D + c, Ls > 0.f ? acc / Ls : 0.f);
  }
  if (lane == 0 && p.lse) p.lse[row] = (Ls > 0.f ? M + fast_log2(Ls) : -INFINITY) * 0.69314718055994531f;
}

// ----------------------------------------------------------------------------- launchers

template <typename T, int D>
static hipError_t launch_decode_t(const PlainParams& p, int waves, bool trace, hipStream_t s) {
  dim3 grid(p.n_splits, p.hq, p.n_rows);
  if (waves == 2) {
    if (trace) hipLaunchKernelGGL((decode_kernel<T, D, 2, true>), grid, dim3(128), 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<T, D, 2, false>), grid, dim3(128), 0, s, p);
  } else if (waves == 8) {
    if (trace) hipLaunchKernelGGL((decode_kernel<T, D, 8, true>), grid, dim3(512), 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<T, D, 8, false>), grid, dim3(512), 0, s, p);
  } else {
    if (trace) hipLaunchKernelGGL((decode_kernel<T, D, 4, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<T, D, 4, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const PlainParams& p, int dtype, int head_dim, int waves, bool trace, hipStream_t s) {
  if (dtype == 0) {
    if (head_dim == 64) return launch_decode_t<float, 64>(p, waves, trace, s);
    if (head_dim == 96) return launch_decode_t<float, 96>(p, waves, trace, s);
    if (head_dim == 128) return launch_decode_t<float, 128>(p, waves, trace, s);
  } else {
    if (head_dim == 64) return launch_decode_t<bf16, 64>(p, waves, trace, s);
    if (head_dim == 96) return launch_decode_t<bf16, 96>(p, waves, trace, s);
    if (head_dim == 128) return launch_decode_t<bf16, 128>(p, waves, trace, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, hipStream_t s) {
  dim3 grid((p.n_rows + 1) / 2);
  if (dtype == 0) {
    if (head_dim == 64) hipLaunchKernelGGL((merge_kernel<float, 64>), grid, dim3(128), 0, s, p);
    else if (head_dim == 96) hipLaunchKernelGGL((merge_kernel<float, 96>), grid, dim3(128), 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<float, 128>), grid, dim3(128), 0, s, p);
  } else {
    if (head_dim == 64) hipLaunchKernelGGL((merge_kernel<bf16, 64>), grid, dim3(128), 0, s, p);
    else if (head_dim == 96) hipLaunchKernelGGL((merge_kernel<bf16, 96>), grid, dim3(128), 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<bf16, 128>), grid, dim3(128), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace lkv
