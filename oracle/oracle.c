/*
 * Plain fp64 reference for loop-aware attention over a looped model's
 * multi-plane KV cache.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this.  It shares no code with the HIP library:
 * every routine here is the textbook definition written out in fp64, one row at
 * a time, with no tiling, paging, online softmax or reordering.
 *
 * Sources (page, section / equation):
 *   [RIPE]   "Prefix Keys and Values Matter Late: RIPE Caching for
 *            Self-Speculative Decoding in Looped Language Models":
 *            Sec. 2 (cache policies pi(r,t,j), full and deepest-plane caches),
 *            Sec. 4 Eq. (9) (RIPE policy), Algorithm 1 and Proposition 1
 *            (block tokens read their own plane).
 *   [LoopKV] "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
 *            Transformers": Sec. 3.1 (KIVI-style codes: K per channel, V per
 *            token, groups of 32 with fp16 scale and zero), Sec. 3.2 (a shared
 *            cell reads the final loop's history with its own query; sink and
 *            window stay its own and exact), Sec. 3.3 (bit-plane V; a cold token
 *            decodes to 4*hi + 1.5; seed m0 = largest sink score), Sec. 3.4 and
 *            App. E Algorithm 1 (partials merged exactly by log-sum-exp).
 *
 * Conventions: loops are 0-based (deepest = n_loops - 1); a row's cache holds
 * positions 0..L-1 including its query block [t0, L); the query at position t
 * sees keys j <= t; the score scale is 1/sqrt(d).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_FULL 0
#define ORACLE_RIPE 1

#define CELL_INT4 1
#define CELL_INT2 2
#define CELL_SHARED 3

/*
 * Plane of key position j read at loop `loop` by the query at position t whose
 * block starts at t0 ([RIPE] Sec. 2 policy pi, Eq. (9)).
 *  - block positions j >= t0 read the loop's own plane (the block pass computes
 *    plane r of earlier block tokens before loop r attends; proof of Prop. 1);
 *  - FULL: every position reads the own plane (pi = r);
 *  - RIPE: own plane if t - j <= W, else the deepest plane.  W = 0 is the
 *    deepest-plane cache (pi = R) for every cached position.
 */
int oracle_plane(int policy, int loop, int n_loops, int64_t t, int64_t t0, int64_t j, int64_t window) {
  if (j >= t0) return loop;
  if (policy == ORACLE_FULL) return loop;
  return (t - j <= window) ? loop : n_loops - 1;
}

static double dot(const double* a, const double* b, int d) {
  double s = 0.0;
  for (int c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

/*
 * One attention row: softmax(q K_view^T / sqrt(d)) V_view over keys 0..t, where
 * K_view/V_view take each position from the plane oracle_plane() names.
 * k_own/v_own hold the loop's own plane, k_deep/v_deep the deepest plane, both
 * [L][d] row-major.  Writes out[d], *lse (natural log), and plane_trace[j]
 * (plane read at j, or -1 for j > t) when plane_trace is not NULL.
 */
void oracle_attend_row(int d, int L, int t, int t0, const double* q, const double* k_own,
                       const double* v_own, const double* k_deep, const double* v_deep, int policy,
                       int loop, int n_loops, int window, double* out, double* lse,
                       int32_t* plane_trace) {
  const double scale = 1.0 / sqrt((double)d);
  double* s = (double*)malloc(sizeof(double) * (size_t)(t + 1));
  double m = -INFINITY;
  for (int j = 0; j <= t; ++j) {
    const int p = oracle_plane(policy, loop, n_loops, t, t0, j, window);
    const double* k = (p == loop ? k_own : k_deep) + (size_t)j * d;
    s[j] = dot(q, k, d) * scale;
    if (s[j] > m) m = s[j];
    if (plane_trace) plane_trace[j] = p;
  }
  if (plane_trace)
    for (int j = t + 1; j < L; ++j) plane_trace[j] = -1;
  double l = 0.0;
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  for (int j = 0; j <= t; ++j) {
    const int p = oracle_plane(policy, loop, n_loops, t, t0, j, window);
    const double* v = (p == loop ? v_own : v_deep) + (size_t)j * d;
    const double e = exp(s[j] - m);
    l += e;
    for (int c = 0; c < d; ++c) out[c] += e * v[c];
  }
  for (int c = 0; c < d; ++c) out[c] /= l;
  *lse = m + log(l);
  free(s);
}

/*
 * Many independent rows (OpenMP over rows).  Row i uses q + i*d and the
 * [L][d] planes at offset i*L*d of each array; t, t0 and loop per row.
 */
void oracle_attend_rows(int n_rows, int d, int L, const int32_t* t, const int32_t* t0,
                        const int32_t* loop, const double* q, const double* k_own,
                        const double* v_own, const double* k_deep, const double* v_deep,
                        int policy, int n_loops, int window, double* out, double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n_rows; ++i) {
    const size_t off = (size_t)i * L * d;
    oracle_attend_row(d, L, t[i], t0[i], q + (size_t)i * d, k_own + off, v_own + off, k_deep + off,
                      v_deep + off, policy, loop[i], n_loops, window, out + (size_t)i * d, lse + i, NULL);
  }
}

/*
 * Split-K partials of one row ([LoopKV] Sec. 3.4: blocks of a row each take a
 * share of the history; App. E Alg. 1).  The visible keys 0..t span
 * n = ceil((t+1)/page) pages; chunk c covers pages [floor(c*n/S), floor((c+1)*n/S)).
 * Chunk c's partial is its own softmax: m_c = max score, l_c = sum exp(s - m_c),
 * o_c = sum exp(s - m_c) v / l_c.  An empty chunk is (0, -inf, 0).
 */
void oracle_split_partials(int d, int L, int t, int t0, const double* q, const double* k_own,
                           const double* v_own, const double* k_deep, const double* v_deep,
                           int policy, int loop, int n_loops, int window, int page, int n_splits,
                           double* o_parts, double* m_parts, double* l_parts) {
  (void)L;
  const double scale = 1.0 / sqrt((double)d);
  const int n_pages = (t + 1 + page - 1) / page;
  for (int c = 0; c < n_splits; ++c) {
    const int p0 = (int)((int64_t)c * n_pages / n_splits);
    const int p1 = (int)((int64_t)(c + 1) * n_pages / n_splits);
    int j0 = p0 * page, j1 = p1 * page;
    if (j1 > t + 1) j1 = t + 1;
    double* o = o_parts + (size_t)c * d;
    for (int x = 0; x < d; ++x) o[x] = 0.0;
    double m = -INFINITY;
    for (int j = j0; j < j1; ++j) {
      const int p = oracle_plane(policy, loop, n_loops, t, t0, j, window);
      const double s = dot(q, (p == loop ? k_own : k_deep) + (size_t)j * d, d) * scale;
      if (s > m) m = s;
    }
    double l = 0.0;
    for (int j = j0; j < j1; ++j) {
      const int p = oracle_plane(policy, loop, n_loops, t, t0, j, window);
      const double s = dot(q, (p == loop ? k_own : k_deep) + (size_t)j * d, d) * scale;
      const double e = exp(s - m);
      const double* v = (p == loop ? v_own : v_deep) + (size_t)j * d;
      l += e;
      for (int x = 0; x < d; ++x) o[x] += e * v[x];
    }
    if (l > 0.0)
      for (int x = 0; x < d; ++x) o[x] /= l;
    m_parts[c] = m;
    l_parts[c] = l;
  }
}

/*
 * Exact log-sum-exp merge of partials ([LoopKV] Sec. 3.4, "the last block of a
 * row merges all partials by log-sum-exp"): m* = max m_c,
 * l* = sum l_c exp(m_c - m*), o = sum o_c l_c exp(m_c - m*) / l*, lse = m* + ln l*.
 */
void oracle_lse_merge(int n_parts, int d, const double* o_parts, const double* m_parts,
                      const double* l_parts, double* out, double* lse) {
  double m = -INFINITY;
  for (int c = 0; c < n_parts; ++c)
    if (l_parts[c] > 0.0 && m_parts[c] > m) m = m_parts[c];
  double l = 0.0;
  for (int x = 0; x < d; ++x) out[x] = 0.0;
  for (int c = 0; c < n_parts; ++c) {
    if (!(l_parts[c] > 0.0)) continue;
    const double w = l_parts[c] * exp(m_parts[c] - m);
    l += w;
    for (int x = 0; x < d; ++x) out[x] += w * o_parts[(size_t)c * d + x];
  }
  for (int x = 0; x < d; ++x) out[x] /= l;
  *lse = m + log(l);
}

/*
 * One decode row of a LoopKV-style quantised cell ([LoopKV] Sec. 3.1-3.4).
 *
 * Regions of the row's L positions (query at t = L-1):
 *   sink S = [0, sink) and tail T = [L-tail, L): exact keys/values of the
 *     cell's own loop (k_near/v_near, [L][d], only S and T rows are read);
 *   far F = [sink, L-tail): codes.  A SHARED cell passes the final loop's codes
 *     (pointer redirection); the caller does that, the arithmetic is the same.
 * Dequantisation:
 *   K per channel over 32-token groups g = (j - sink)/32:
 *     k_hat[j][c] = kz[g][c] + ks[g][c] * kc[j-sink][c];
 *   V per token over 32-channel groups:
 *     INT2: v_hat = vz[j][c/32] + vs[j][c/32] * vc;
 *     INT4 / SHARED (bit planes hi = c >> 2, lo = c & 3): a hot token reads
 *       both planes (4*hi + lo = c), a cold token only hi and decodes to the
 *       bucket midpoint 4*hi + 1.5.
 * Seed: m0 = max score over the sink keys ([LoopKV] Sec. 3.3, footnote 9).
 * Hot test of far token j (s in natural logit units, ties hot); INT2 cells
 * have no lo plane and no test (hot_bits are written as 1):
 *   rule 0 (fixed):   s_j >= m0 - thr;
 *   rule 1 (running, [LoopKV] Sec. 3.3 and App. E Algorithm 1): the far history's
 *     32-token pages are shared out to n_splits far blocks, block c taking pages
 *     [floor(c n / S), floor((c+1) n / S)); each block walks its pages in order,
 *     and after reading page p's keys its running maximum m is the largest score
 *     of its pages up to and including p; token j of page p is hot iff
 *     s_j >= max(m, m0) - thr, where thr = tau ln 2 is passed in.
 * Softmax over S, F and T as in oracle_attend_row.  Writes out[d], *lse,
 * hot_bits[L-tail-sink] (0/1), thr_used[L-tail-sink] (the threshold each far
 * token was tested against, or NaN for INT2; may be NULL) and returns the number
 * of cold far tokens.
 */
int oracle_cell_row_rule(int d, int L, int sink, int tail, int kind, const double* q,
                         const double* k_near, const double* v_near, const uint8_t* kc,
                         const double* ks, const double* kz, const uint8_t* vc, const double* vs,
                         const double* vz, int rule, double thr_offset, int n_splits, double* out,
                         double* lse, uint8_t* hot_bits, double* thr_used) {
  const double scale = 1.0 / sqrt((double)d);
  const int n_far = L - tail - sink;
  const int n_grp = d / 32;
  double* s = (double*)malloc(sizeof(double) * (size_t)L);
  double* kh = (double*)malloc(sizeof(double) * (size_t)d);
  double m0 = -INFINITY;
  for (int j = 0; j < sink; ++j) {
    s[j] = dot(q, k_near + (size_t)j * d, d) * scale;
    if (s[j] > m0) m0 = s[j];
  }
  for (int j = L - tail; j < L; ++j) s[j] = dot(q, k_near + (size_t)j * d, d) * scale;
  for (int f = 0; f < n_far; ++f) {
    const int g = f / 32;
    for (int c = 0; c < d; ++c)
      kh[c] = kz[(size_t)g * d + c] + ks[(size_t)g * d + c] * (double)kc[(size_t)f * d + c];
    s[sink + f] = dot(q, kh, d) * scale;
  }
  const int masked = (kind == CELL_INT4 || kind == CELL_SHARED);
  int n_cold = 0;
  if (!masked || rule == 0) {
    const double thr = m0 - thr_offset;
    for (int f = 0; f < n_far; ++f) {
      const int hot = masked ? (s[sink + f] >= thr) : 1;
      hot_bits[f] = (uint8_t)hot;
      if (thr_used) thr_used[f] = masked ? thr : NAN;
      n_cold += !hot;
    }
  } else {
    const int n_pages = (n_far + 31) / 32;
    for (int c = 0; c < n_splits; ++c) {
      const int p0 = (int)((int64_t)c * n_pages / n_splits), p1 = (int)((int64_t)(c + 1) * n_pages / n_splits);
      double m = -INFINITY;
      for (int p = p0; p < p1; ++p) {
        const int f0 = 32 * p, f1 = 32 * p + 32 < n_far ? 32 * p + 32 : n_far;
        for (int f = f0; f < f1; ++f)
          if (s[sink + f] > m) m = s[sink + f];
        const double thr = (m > m0 ? m : m0) - thr_offset;
        for (int f = f0; f < f1; ++f) {
          const int hot = s[sink + f] >= thr;
          hot_bits[f] = (uint8_t)hot;
          if (thr_used) thr_used[f] = thr;
          n_cold += !hot;
        }
      }
    }
  }
  double m = -INFINITY;
  for (int j = 0; j < L; ++j)
    if (s[j] > m) m = s[j];
  double l = 0.0;
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  for (int j = 0; j < L; ++j) {
    const double e = exp(s[j] - m);
    l += e;
    if (j < sink || j >= L - tail) {
      for (int c = 0; c < d; ++c) out[c] += e * v_near[(size_t)j * d + c];
      continue;
    }
    const int f = j - sink;
    for (int c = 0; c < d; ++c) {
      const int code = vc[(size_t)f * d + c];
      double chat;
      if (!masked) chat = (double)code;
      else if (hot_bits[f]) chat = (double)code;
      else chat = 4.0 * (double)(code >> 2) + 1.5;
      const double v = vz[(size_t)f * n_grp + c / 32] + vs[(size_t)f * n_grp + c / 32] * chat;
      out[c] += e * v;
    }
  }
  for (int c = 0; c < d; ++c) out[c] /= l;
  *lse = m + log(l);
  free(kh);
  free(s);
  return n_cold;
}

/* The fixed rule (s_j >= m0 - thr_offset) of oracle_cell_row_rule. */
int oracle_cell_row(int d, int L, int sink, int tail, int kind, const double* q, const double* k_near,
                    const double* v_near, const uint8_t* kc, const double* ks, const double* kz,
                    const uint8_t* vc, const double* vs, const double* vz, double thr_offset, double* out,
                    double* lse, uint8_t* hot_bits) {
  return oracle_cell_row_rule(d, L, sink, tail, kind, q, k_near, v_near, kc, ks, kz, vc, vs, vz, 0, thr_offset, 1,
                              out, lse, hot_bits, NULL);
}

/*
 * The window-exit codec ([LoopKV] Sec. 3.1: KIVI-style codes, keys per channel and
 * values per token in groups of 32 with an fp16 scale and zero; Sec. 3.3: the
 * INT4 value code c is stored as hi = c >> 2 and lo = c & 3).  This is the
 * encoder that turns one far page of exact keys and values into codes.
 *
 * Per group of values x (a key channel over the page's tokens, or a token's 32
 * consecutive value channels):
 *   mn, mx = smallest and largest x (exact);
 *   sigma = (mx - mn) / (2^b - 1) in fp32 (one IEEE division), zero = mn;
 *   both rounded to fp16, nearest-even: s16, z16;
 *   c = clamp(rint((x - z16) / s16), 0, 2^b - 1) in fp32 (one subtraction and
 *   one IEEE division, each rounded; rint rounds half to even); c = 0 if s16 = 0.
 * The arithmetic is fp32 because the method stores fp16 metadata computed from
 * fp32 statistics; no operation is fused.
 */
static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> fp16 bits, IEEE round to nearest even (normal, subnormal, overflow to inf). */
uint16_t oracle_f16_from_f32(float f) {
  const uint32_t u = f32_bits(f);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (a > 0x7F800000u ? 0x200u : 0u));
  const int e = (int)(a >> 23) - 127; /* unbiased exponent */
  uint32_t m = (a & 0x7FFFFFu) | (a >= 0x00800000u ? 0x800000u : 0u);
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  /* value = m * 2^(e - 23); fp16 quantum is 2^-24 for subnormals, 2^(e - 10) for normals */
  const int q = e < -14 ? -24 : e - 10;
  const int shift = q - (e - 23); /* bits of m below the fp16 quantum */
  uint32_t h;
  if (shift >= 32) {
    h = 0;
  } else {
    const uint32_t kept = m >> shift, rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1);
    h = kept + ((rem > half || (rem == half && (kept & 1u))) ? 1u : 0u);
  }
  /* h counts quanta: assemble, letting a carry roll into the exponent */
  uint32_t out;
  if (e < -14) {
    out = h; /* subnormal, or the smallest normal after rounding up */
  } else {
    out = ((uint32_t)(e + 15) << 10) + (h - 0x400u);
  }
  if (out >= 0x7C00u) out = 0x7C00u;
  return (uint16_t)(sign | out);
}

float oracle_f32_from_f16(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  if (e == 0) {
    const float v = (float)m * bits_f32(0x33800000u); /* m * 2^-24, exact */
    return sign ? -v : v;
  }
  if (e == 31) return bits_f32(sign | 0x7F800000u | (m << 13));
  return bits_f32(sign | ((e + 112u) << 23) | (m << 13));
}

static void encode_group(const float* x, int n, int stride, int levels, uint8_t* c, int cstride,
                         uint16_t* s16, uint16_t* z16) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; ++i) {
    const float v = x[(size_t)i * stride];
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  const float sigma = (mx - mn) / (float)levels;
  *s16 = oracle_f16_from_f32(sigma);
  *z16 = oracle_f16_from_f32(mn);
  const float s = oracle_f32_from_f16(*s16), z = oracle_f32_from_f16(*z16);
  for (int i = 0; i < n; ++i) {
    float q = 0.0f;
    if (s != 0.0f) {
      const float t = (x[(size_t)i * stride] - z) / s;
      q = rintf(t);
      if (q < 0.0f) q = 0.0f;
      if (q > (float)levels) q = (float)levels;
    }
    c[(size_t)i * cstride] = (uint8_t)q;
  }
}

/*
 * Encode one far page of one head: k, v are [n_tok][d] (exact values, here
 * bf16 widened to fp32), n_tok <= 32 valid tokens, bits 4 or 2.
 * Outputs: kc, vc [n_tok][d] codes; kmeta [d][2] (scale, zero) fp16 bits per key
 * channel; vmeta [n_tok][d/32][2] per token and 32-channel group.
 */
void oracle_kivi_encode(int n_tok, int d, int bits, const float* k, const float* v, uint8_t* kc,
                        uint16_t* kmeta, uint8_t* vc, uint16_t* vmeta) {
  const int levels = (1 << bits) - 1;
  for (int ch = 0; ch < d; ++ch)
    encode_group(k + ch, n_tok, d, levels, kc + ch, d, &kmeta[2 * ch], &kmeta[2 * ch + 1]);
  for (int t = 0; t < n_tok; ++t)
    for (int g = 0; g < d / 32; ++g) {
      uint16_t* m = &vmeta[((size_t)t * (d / 32) + g) * 2];
      encode_group(v + (size_t)t * d + 32 * g, 32, 1, levels, vc + (size_t)t * d + 32 * g, 1, &m[0], &m[1]);
    }
}

/* Threads the row-parallel routines use (OpenMP), for reporting. */
int oracle_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}

/* Sets the threads the row-parallel routines use from here on (for timing them on one
   core); returns the previous setting.  No arithmetic depends on it. */
int oracle_set_threads(int n) {
  const int prev = omp_get_max_threads();
  omp_set_num_threads(n > 0 ? n : 1);
  return prev;
}
