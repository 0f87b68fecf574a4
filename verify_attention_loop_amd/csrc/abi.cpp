// C-ABI of the loop-aware attention library: the paged plane allocator, its
// block tables, cell descriptors and argument checking, and the kernel launches.
//
// Host bookkeeping only touches host memory; device work (copies, table uploads,
// kernels) happens in lkv_append_plane / lkv_append_coded / lkv_encode_pages /
// lkv_attend on the caller's stream.  The library never allocates device memory,
// and every device write it issues is a kernel (block-table rows travel as kernel
// arguments; trace buffers are cleared by a fill kernel), so the calls can be
// captured into a graph and never copy from pageable host memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "loopattn.h"
#include "launch.hpp"
#include "params.hpp"

namespace lkv {
hipError_t launch_decode(const PlainParams& p, int dtype, int head_dim, int waves, bool trace, hipStream_t s,
                         const LaunchEvents& ev);
hipError_t launch_verify(const PlainParams& p, int dtype, int head_dim, int waves, bool trace, hipStream_t s,
                         const LaunchEvents& ev);
int verify_heads_per_wg(int hq, int hkv, int q_len, int head_dim);
hipError_t launch_gqa_decode(const PlainParams& p, int dtype, int head_dim, int waves, bool trace, hipStream_t s,
                             const LaunchEvents& ev);
hipError_t launch_merge(const MergeParams& p, int dtype, int head_dim, hipStream_t s);
hipError_t launch_append(const CopyParams& p, int dtype, int head_dim, hipStream_t s);
hipError_t launch_fill(void* dst, uint64_t n_bytes, uint32_t value, hipStream_t s);
hipError_t launch_table_write(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s);
hipError_t launch_cell(const CellParams& p, int head_dim, int waves, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_probe_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_pack_codes(const PackParams& p, int head_dim, hipStream_t s);
hipError_t launch_encode_pages(const EncodeParams& p, int head_dim, hipStream_t s);
hipError_t launch_read_codes(const PackParams& p, int head_dim, void* k_codes, void* k_meta, void* v_codes,
                             void* v_meta, hipStream_t s);
uint64_t code_page_bytes(int hkv, int head_dim, int bits);
}  // namespace lkv

using namespace lkv;

namespace {

// SplitMix64 (Steele, Lea, Flood 2014) for the seeded page permutation.
inline uint64_t splitmix64(uint64_t& state) {
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct FreeList {
  std::vector<int32_t> stack;  // back() is handed out next
  int64_t total = 0;

  void init(int64_t n, uint64_t seed) {
    total = n;
    stack.resize((size_t)n);
    for (int64_t i = 0; i < n; ++i) stack[(size_t)i] = (int32_t)(n - 1 - i);
    if (seed != 0 && n > 1) {  // Fisher-Yates with SplitMix64 draws
      uint64_t st = seed;
      for (int64_t i = n - 1; i > 0; --i) {
        const int64_t j = (int64_t)(splitmix64(st) % (uint64_t)(i + 1));
        std::swap(stack[(size_t)i], stack[(size_t)j]);
      }
    }
  }
  int64_t available() const { return (int64_t)stack.size(); }
  int64_t in_use() const { return total - (int64_t)stack.size(); }
  int32_t pop() {
    const int32_t v = stack.back();
    stack.pop_back();
    return v;
  }
  void push(int32_t v) { stack.push_back(v); }
};

// Block table of one (layer, plane) or (layer, loop) code cell: per sequence slot,
// `ring` entries; logical page p lives in entry p % ring.
struct Table {
  int32_t ring = 0;
  bool window_ring = false;      // RIPE non-deepest plane: entries recycle as the window slides
  size_t dev_off = 0;            // byte offset in the meta arena
  std::vector<int32_t> phys;     // [slot * ring + e]: physical page or -1
  std::vector<int32_t> owner;    // logical page held by entry e, or -1
  std::vector<uint8_t> dirty;    // per sequence slot: host row differs from the device copy
  std::vector<int32_t> hi;       // per sequence slot: positions [.., hi) written
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int elem_bytes(const lkv_config& c) { return c.kv_dtype == LKV_DTYPE_F32 ? 4 : 2; }

}  // namespace

struct lkv_cache {
  lkv_config cfg{};
  lkv_arenas ar{};
  int device = 0;
  uint64_t page_bytes = 0, code4_bytes = 0, code2_bytes = 0;
  int32_t max_pages = 0, ring_pages = 0, max_code_pages = 0;
  FreeList pages, codes4, codes2;
  std::vector<Table> tabs;   // [layer * n_loops + plane]
  std::vector<Table> ctabs;  // [layer * n_loops + loop], quant only
  std::vector<int8_t> plan;
  bool plan_set = false;
  struct Seq {
    bool live = false;
    int32_t len = 0;
    int32_t committed = 0;
  };
  std::vector<Seq> seqs;
  std::string err;

  lkv_status fail(lkv_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    err = buf;
    return s;
  }
  Table& tab(int layer, int plane) { return tabs[(size_t)layer * cfg.n_loops + plane]; }
  const Table& tab(int layer, int plane) const { return tabs[(size_t)layer * cfg.n_loops + plane]; }
  Table& ctab(int layer, int loop) { return ctabs[(size_t)layer * cfg.n_loops + loop]; }
  int deepest() const { return cfg.n_loops - 1; }
  bool live(int32_t s) const { return s >= 0 && s < cfg.max_seqs && seqs[(size_t)s].live; }
};

namespace {

lkv_status check_config(const lkv_config* c, std::string* why) {
  auto bad = [&](const char* m) {
    if (why) *why = m;
    return LKV_EINVAL;
  };
  if (!c) return bad("config is NULL");
  if (c->n_layers < 1 || c->n_loops < 1) return bad("n_layers and n_loops must be >= 1");
  if (c->n_heads_q < 1 || c->n_heads_kv < 1 || c->n_heads_q % c->n_heads_kv) return bad("bad head counts");
  if (c->head_dim != 64 && c->head_dim != 96 && c->head_dim != 128 && c->head_dim != 256)
    return bad("head_dim must be 64, 96, 128 or 256");
  if (c->head_dim == 256 && c->kv_dtype != LKV_DTYPE_BF16) return bad("head_dim 256 is built for bf16 caches");
  if (c->page_size != LKV_PAGE_TOKENS) return bad("page_size must be 16");
  if (c->kv_dtype != LKV_DTYPE_F32 && c->kv_dtype != LKV_DTYPE_BF16) return bad("bad kv_dtype");
  if (c->policy != LKV_POLICY_FULL && c->policy != LKV_POLICY_RIPE) return bad("bad policy");
  if (c->window < 0) return bad("window must be >= 0");
  if (c->max_seqs < 1 || c->max_len < 1) return bad("max_seqs and max_len must be >= 1");
  if (c->max_block < 1 || c->max_block > kMaxBlock) return bad("max_block must be in 1..16");
  if (c->quant != 0 && c->quant != 1) return bad("quant must be 0 or 1");
  if (c->quant) {
    if (c->kv_dtype != LKV_DTYPE_BF16) return bad("quantised cells keep bf16 sink and tail");
    if (c->policy != LKV_POLICY_FULL) return bad("quantised cells use the full-cache policy");
    if (c->sink < 1 || c->sink > 4 * kPage || c->tail < 0) return bad("quantised cells need 1 <= sink <= 64, tail >= 0");
    if (c->head_dim % 32) return bad("quantised cells need head_dim % 32 == 0");
    if (c->head_dim != 128) return bad("quantised cells are built for head_dim 128");
  }
  return LKV_OK;
}

struct Layout {
  uint64_t page_bytes, code4_bytes, code2_bytes;
  int32_t max_pages, ring_pages, max_code_pages;
  size_t meta_bytes;
};

Layout layout_of(const lkv_config& c) {
  Layout L{};
  L.page_bytes = 2ull * c.n_heads_kv * kPage * c.head_dim * elem_bytes(c);
  L.max_pages = (c.max_len + kPage - 1) / kPage;
  L.ring_pages = std::min(L.max_pages, (c.window + c.max_block + kPage - 1) / kPage + 1);
  if (c.quant) {
    L.code4_bytes = code_page_bytes(c.n_heads_kv, c.head_dim, 4);
    L.code2_bytes = code_page_bytes(c.n_heads_kv, c.head_dim, 2);
    const int far = std::max(0, c.max_len - c.sink - c.tail);
    L.max_code_pages = std::max(1, (far + kCodePage - 1) / kCodePage);
  }
  size_t m = 0;
  for (int l = 0; l < c.n_layers; ++l)
    for (int p = 0; p < c.n_loops; ++p) {
      const bool ring = c.policy == LKV_POLICY_RIPE && !c.quant && p < c.n_loops - 1;
      m += align256((size_t)c.max_seqs * (ring ? L.ring_pages : L.max_pages) * 4);
    }
  if (c.quant) m += (size_t)c.n_layers * c.n_loops * align256((size_t)c.max_seqs * L.max_code_pages * 4);
  L.meta_bytes = m;
  return L;
}

lkv_status hip_fail(lkv_cache* c, hipError_t e, const char* what) {
  return c->fail(LKV_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* lkv_status_str(lkv_status s) {
  switch (s) {
    case LKV_OK: return "ok";
    case LKV_EINVAL: return "invalid argument";
    case LKV_ENOMEM: return "out of pages or workspace";
    case LKV_ESTATE: return "cache state does not allow the call";
    case LKV_EWINDOW: return "outside the RIPE window ring";
    case LKV_EDEVICE: return "device error";
    case LKV_EUNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* lkv_last_error(const lkv_cache* c) { return c ? c->err.c_str() : "NULL handle"; }

lkv_status lkv_sizes(const lkv_config* cfg, lkv_size_info* out) {
  if (!out || check_config(cfg, nullptr) != LKV_OK) return LKV_EINVAL;
  const Layout L = layout_of(*cfg);
  out->page_bytes = L.page_bytes;
  out->code4_page_bytes = L.code4_bytes;
  out->code2_page_bytes = L.code2_bytes;
  out->meta_bytes = L.meta_bytes;
  return LKV_OK;
}

lkv_status lkv_create(const lkv_config* cfg, const lkv_arenas* ar, int device, lkv_cache** out) {
  if (!out || !ar) return LKV_EINVAL;
  *out = nullptr;
  if (check_config(cfg, nullptr) != LKV_OK) return LKV_EINVAL;
  const Layout L = layout_of(*cfg);
  if (!ar->meta || ar->meta_bytes < L.meta_bytes) return LKV_ENOMEM;
  if (ar->pages_bytes && !ar->pages) return LKV_EINVAL;
  const int64_t n_pages = (int64_t)(ar->pages_bytes / L.page_bytes);
  int64_t n4 = 0, n2 = 0;
  if (cfg->quant) {
    if ((ar->codes4_bytes && !ar->codes4) || (ar->codes2_bytes && !ar->codes2)) return LKV_EINVAL;
    n4 = (int64_t)(ar->codes4_bytes / L.code4_bytes);
    n2 = (int64_t)(ar->codes2_bytes / L.code2_bytes);
  }
  if (n_pages > INT32_MAX || n4 > INT32_MAX || n2 > INT32_MAX) return LKV_EINVAL;
  lkv_cache* c = new lkv_cache();
  c->cfg = *cfg;
  c->ar = *ar;
  c->device = device;
  c->page_bytes = L.page_bytes;
  c->code4_bytes = L.code4_bytes;
  c->code2_bytes = L.code2_bytes;
  c->max_pages = L.max_pages;
  c->ring_pages = L.ring_pages;
  c->max_code_pages = L.max_code_pages;
  c->pages.init(n_pages, cfg->shuffle_seed);
  c->codes4.init(n4, cfg->shuffle_seed ? cfg->shuffle_seed + 1 : 0);
  c->codes2.init(n2, cfg->shuffle_seed ? cfg->shuffle_seed + 2 : 0);
  c->seqs.resize((size_t)cfg->max_seqs);
  size_t off = 0;
  c->tabs.resize((size_t)cfg->n_layers * cfg->n_loops);
  for (int l = 0; l < cfg->n_layers; ++l)
    for (int p = 0; p < cfg->n_loops; ++p) {
      Table& T = c->tab(l, p);
      T.window_ring = cfg->policy == LKV_POLICY_RIPE && !cfg->quant && p < cfg->n_loops - 1;
      T.ring = T.window_ring ? L.ring_pages : L.max_pages;
      T.dev_off = off;
      off += align256((size_t)cfg->max_seqs * T.ring * 4);
      T.phys.assign((size_t)cfg->max_seqs * T.ring, -1);
      T.owner.assign((size_t)cfg->max_seqs * T.ring, -1);
      T.dirty.assign((size_t)cfg->max_seqs, 1);
      T.hi.assign((size_t)cfg->max_seqs, 0);
    }
  if (cfg->quant) {
    c->ctabs.resize((size_t)cfg->n_layers * cfg->n_loops);
    for (auto& T : c->ctabs) {
      T.ring = L.max_code_pages;
      T.dev_off = off;
      off += align256((size_t)cfg->max_seqs * T.ring * 4);
      T.phys.assign((size_t)cfg->max_seqs * T.ring, -1);
      T.owner.assign((size_t)cfg->max_seqs * T.ring, -1);
      T.dirty.assign((size_t)cfg->max_seqs, 1);
      T.hi.assign((size_t)cfg->max_seqs, 0);
    }
    c->plan.assign((size_t)cfg->n_layers * cfg->n_loops, LKV_CELL_INT4);
  }
  *out = c;
  return LKV_OK;
}

lkv_status lkv_destroy(lkv_cache* c) {
  delete c;
  return LKV_OK;
}

lkv_status lkv_add_seq(lkv_cache* c, int32_t* seq_out) {
  if (!c || !seq_out) return LKV_EINVAL;
  for (int s = 0; s < c->cfg.max_seqs; ++s)
    if (!c->seqs[(size_t)s].live) {
      c->seqs[(size_t)s] = lkv_cache::Seq{true, 0, 0};
      *seq_out = s;
      return LKV_OK;
    }
  return c->fail(LKV_ENOMEM, "all %d sequence slots are in use", c->cfg.max_seqs);
}

static void release_row(lkv_cache* c, Table& T, FreeList& fl, int32_t seq, int32_t first_page_from) {
  for (int e = 0; e < T.ring; ++e) {
    const size_t i = (size_t)seq * T.ring + e;
    if (T.owner[i] >= 0 && T.owner[i] >= first_page_from) {
      fl.push(T.phys[i]);
      T.phys[i] = -1;
      T.owner[i] = -1;
      T.dirty[(size_t)seq] = 1;
    }
  }
}

lkv_status lkv_free_seq(lkv_cache* c, int32_t seq) {
  if (!c) return LKV_EINVAL;
  if (!c->live(seq)) return c->fail(LKV_EINVAL, "sequence %d is not live", seq);
  for (auto& T : c->tabs) {
    release_row(c, T, c->pages, seq, 0);
    T.hi[(size_t)seq] = 0;
  }
  for (size_t k = 0; k < c->ctabs.size(); ++k) {
    Table& T = c->ctabs[k];
    FreeList& fl = c->plan[k] == LKV_CELL_INT2 ? c->codes2 : c->codes4;
    release_row(c, T, fl, seq, 0);
    T.hi[(size_t)seq] = 0;
  }
  c->seqs[(size_t)seq] = lkv_cache::Seq{};
  return LKV_OK;
}

// Reserve pages for positions [pos0, pos0 + n) of (seq, layer, plane).  On success
// `touched` receives (logical page, physical page, newly handed out) per page.
struct Touched {
  int32_t logical, phys;
  bool fresh;
};

// Far positions of (seq, layer, loop) already held as codes: those of the cell's source
// (its own codes, or the final loop's for a shared cell); 0 before a plan is set.
static int32_t encoded_far(const lkv_cache* c, int32_t seq, int32_t layer, int32_t loop) {
  if (!c->cfg.quant || !c->plan_set) return 0;
  const int R = c->cfg.n_loops;
  const int src = c->plan[(size_t)layer * R + loop] == LKV_CELL_SHARED ? R - 1 : loop;
  return c->ctabs[(size_t)layer * R + src].hi[(size_t)seq];
}

static lkv_status reserve_impl(lkv_cache* c, int32_t seq, int32_t layer, int32_t plane, int32_t pos0,
                               int32_t n_tok, std::vector<Touched>* touched) {
  if (!c->live(seq)) return c->fail(LKV_EINVAL, "sequence %d is not live", seq);
  if (layer < 0 || layer >= c->cfg.n_layers) return c->fail(LKV_EINVAL, "layer %d out of range", layer);
  if (plane < 0 || plane >= c->cfg.n_loops) return c->fail(LKV_EINVAL, "plane %d out of range", plane);
  if (pos0 < 0 || n_tok < 1 || (int64_t)pos0 + n_tok > c->cfg.max_len)
    return c->fail(LKV_EINVAL, "positions [%d, %d) outside [0, max_len=%d)", pos0, pos0 + n_tok, c->cfg.max_len);
  Table& T = c->tab(layer, plane);
  const auto& S = c->seqs[(size_t)seq];
  const int32_t hi = T.hi[(size_t)seq];
  const int32_t lo_win = std::max(0, S.committed - c->cfg.window);
  if (c->cfg.quant) {
    // The exact bf16 plane holds the sink and the tail; positions that left the tail
    // live as codes.  No gap, except that a far history supplied as code pages may be
    // skipped after the sink; positions already encoded cannot be written again.
    if (pos0 > hi && !(hi <= c->cfg.sink && pos0 >= c->cfg.sink))
      return c->fail(LKV_ESTATE, "gap: plane %d of seq %d holds positions up to %d, append starts at %d", plane, seq,
                     hi, pos0);
    const int32_t enc = encoded_far(c, seq, layer, plane);
    if (enc > 0 && pos0 < c->cfg.sink + enc && pos0 + n_tok > c->cfg.sink)
      return c->fail(LKV_ESTATE, "positions [%d, %d) of plane %d already left the tail (encoded up to %d)", pos0,
                     pos0 + n_tok, plane, c->cfg.sink + enc);
  } else {
    if (T.window_ring) {
      if (pos0 < lo_win)
        return c->fail(LKV_EWINDOW, "plane %d keeps positions >= %d only (committed %d, window %d); got %d", plane,
                       lo_win, S.committed, c->cfg.window, pos0);
      if (pos0 > std::max(hi, lo_win))
        return c->fail(LKV_ESTATE, "gap: plane %d of seq %d holds positions up to %d, append starts at %d", plane,
                       seq, std::max(hi, lo_win), pos0);
    } else if (pos0 > hi) {
      return c->fail(LKV_ESTATE, "gap: plane %d of seq %d holds positions [0, %d), append starts at %d", plane, seq,
                     hi, pos0);
    }
  }
  const int32_t p_first = pos0 / kPage, p_last = (pos0 + n_tok - 1) / kPage;
  const int32_t n_touch = p_last - p_first + 1;
  if (n_touch > T.ring)
    return c->fail(LKV_EWINDOW, "append spans %d pages but plane %d holds %d per sequence", n_touch, plane, T.ring);
  // Phase 1: check slots and count pages.
  int64_t need = 0, reclaim = 0;
  for (int32_t p = p_first; p <= p_last; ++p) {
    const size_t i = (size_t)seq * T.ring + (size_t)(p % T.ring);
    const int32_t q = T.owner[i];
    if (q == p) continue;
    ++need;
    if (q >= 0) {
      if (T.window_ring && (int64_t)(q + 1) * kPage <= lo_win) ++reclaim;
      else
        return c->fail(LKV_EWINDOW, "window ring of plane %d is full: page %d still holds live positions", plane, q);
    }
  }
  if (need - reclaim > c->pages.available())
    return c->fail(LKV_ENOMEM, "need %lld pages, %lld free", (long long)(need - reclaim),
                   (long long)c->pages.available());
  // Phase 2: commit.
  if (touched) touched->clear();
  for (int32_t p = p_first; p <= p_last; ++p) {
    const size_t i = (size_t)seq * T.ring + (size_t)(p % T.ring);
    bool fresh = false;
    if (T.owner[i] != p) {
      if (T.owner[i] >= 0) c->pages.push(T.phys[i]);
      T.phys[i] = c->pages.pop();
      T.owner[i] = p;
      fresh = true;
      T.dirty[(size_t)seq] = 1;
    }
    if (touched) touched->push_back(Touched{p, T.phys[i], fresh});
  }
  T.hi[(size_t)seq] = std::max(hi, pos0 + n_tok);
  c->seqs[(size_t)seq].len = std::max(S.len, pos0 + n_tok);
  return LKV_OK;
}

lkv_status lkv_reserve(lkv_cache* c, int32_t seq, int32_t layer, int32_t plane, int32_t pos0, int32_t n_tok) {
  if (!c) return LKV_EINVAL;
  return reserve_impl(c, seq, layer, plane, pos0, n_tok, nullptr);
}

lkv_status lkv_append_plane(lkv_cache* c, int32_t seq, int32_t layer, int32_t plane, int32_t pos0, int32_t n_tok,
                            const void* k, const void* v, void* stream) {
  if (!c) return LKV_EINVAL;
  if (!k || !v) return c->fail(LKV_EINVAL, "k and v must not be NULL");
  std::vector<Touched> touched;
  lkv_status st = reserve_impl(c, seq, layer, plane, pos0, n_tok, &touched);
  if (st != LKV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int es = elem_bytes(c->cfg);
  if (c->cfg.poison) {
    const uint32_t nan = es == 4 ? 0x7FC00000u : 0x7FC07FC0u;
    for (const auto& t : touched)
      if (t.fresh) {
        hipError_t e = launch_fill((uint8_t*)c->ar.pages + (uint64_t)t.phys * c->page_bytes, c->page_bytes, nan, s);
        if (e != hipSuccess) return hip_fail(c, e, "poison fill");
      }
  }
  const int64_t row_bytes = (int64_t)c->cfg.n_heads_kv * c->cfg.head_dim * es;
  for (size_t i0 = 0; i0 < touched.size(); i0 += 64) {
    const size_t i1 = std::min(touched.size(), i0 + 64);
    CopyParams P{};
    P.pool = (uint8_t*)c->ar.pages;
    P.page_bytes = c->page_bytes;
    P.hkv = c->cfg.n_heads_kv;
    P.page0 = touched[i0].logical;
    P.n_pages = (int32_t)(i1 - i0);
    for (size_t i = i0; i < i1; ++i) P.phys[i - i0] = touched[i].phys;
    const int32_t a = std::max(pos0, touched[i0].logical * kPage);
    const int32_t b = std::min(pos0 + n_tok, (touched[i1 - 1].logical + 1) * kPage);
    P.pos0 = a;
    P.n_tok = b - a;
    P.k = (const uint8_t*)k + (int64_t)(a - pos0) * row_bytes;
    P.v = (const uint8_t*)v + (int64_t)(a - pos0) * row_bytes;
    hipError_t e = launch_append(P, c->cfg.kv_dtype, c->cfg.head_dim, s);
    if (e != hipSuccess) return hip_fail(c, e, "append kernel");
  }
  return LKV_OK;
}

lkv_status lkv_commit(lkv_cache* c, int32_t seq, int32_t new_len) {
  if (!c) return LKV_EINVAL;
  if (!c->live(seq)) return c->fail(LKV_EINVAL, "sequence %d is not live", seq);
  auto& S = c->seqs[(size_t)seq];
  // Commit is monotone: the window slides forward only.  Moving it back would re-open
  // positions whose ring pages were already returned to the pool.
  if (new_len < S.committed || new_len > S.len)
    return c->fail(LKV_EINVAL, "commit length %d outside [committed %d, len %d]", new_len, S.committed, S.len);
  S.committed = new_len;
  const int32_t lo_win = std::max(0, new_len - c->cfg.window);
  for (auto& T : c->tabs) {
    if (!T.window_ring) continue;
    for (int e = 0; e < T.ring; ++e) {
      const size_t i = (size_t)seq * T.ring + e;
      if (T.owner[i] >= 0 && (int64_t)(T.owner[i] + 1) * kPage <= lo_win) {
        c->pages.push(T.phys[i]);
        T.phys[i] = -1;
        T.owner[i] = -1;
        T.dirty[(size_t)seq] = 1;
      }
    }
  }
  return LKV_OK;
}

lkv_status lkv_truncate(lkv_cache* c, int32_t seq, int32_t new_len) {
  if (!c) return LKV_EINVAL;
  if (!c->live(seq)) return c->fail(LKV_EINVAL, "sequence %d is not live", seq);
  auto& S = c->seqs[(size_t)seq];
  if (new_len < S.committed || new_len > S.len)
    return c->fail(LKV_EINVAL, "truncate length %d outside [committed %d, len %d]", new_len, S.committed, S.len);
  if (c->cfg.quant)
    for (int l = 0; l < c->cfg.n_layers; ++l)
      for (int r = 0; r < c->cfg.n_loops; ++r)
        if (new_len - c->cfg.tail < c->cfg.sink + encoded_far(c, seq, l, r))
          return c->fail(LKV_ESTATE, "truncate to %d would re-open positions that already left the tail", new_len);
  const int32_t first_dead_page = (new_len + kPage - 1) / kPage;
  for (auto& T : c->tabs) {
    release_row(c, T, c->pages, seq, first_dead_page);
    T.hi[(size_t)seq] = std::min(T.hi[(size_t)seq], new_len);
  }
  S.len = new_len;
  return LKV_OK;
}

lkv_status lkv_set_plan(lkv_cache* c, const int8_t* kinds) {
  if (!c) return LKV_EINVAL;
  if (!c->cfg.quant) return c->fail(LKV_ESTATE, "the cache has no quantised cells");
  if (!kinds) return c->fail(LKV_EINVAL, "kinds is NULL");
  for (const auto& T : c->ctabs)
    for (int32_t o : T.owner)
      if (o >= 0) return c->fail(LKV_ESTATE, "the plan is fixed once code pages exist");
  const int R = c->cfg.n_loops;
  for (int l = 0; l < c->cfg.n_layers; ++l)
    for (int r = 0; r < R; ++r) {
      const int8_t k = kinds[(size_t)l * R + r];
      if (k != LKV_CELL_INT4 && k != LKV_CELL_INT2 && k != LKV_CELL_SHARED)
        return c->fail(LKV_EINVAL, "cell (%d, %d): kind %d", l, r, (int)k);
      if (k == LKV_CELL_SHARED && r == R - 1)
        return c->fail(LKV_EINVAL, "the final loop's cell (layer %d) is the source of shared cells", l);
    }
  std::memcpy(c->plan.data(), kinds, c->plan.size());
  c->plan_set = true;
  return LKV_OK;
}

// Checks shared by the code-page calls; on success fills the cell's table, free list,
// arena, page size and bit width.
static lkv_status code_cell(lkv_cache* c, int32_t seq, int32_t layer, int32_t loop, int32_t page0, int32_t n_pages,
                            Table** T, FreeList** fl, uint8_t** arena, uint64_t* cpb, int* bits) {
  if (!c->cfg.quant) return c->fail(LKV_ESTATE, "the cache has no quantised cells");
  if (!c->plan_set) return c->fail(LKV_ESTATE, "lkv_set_plan first");
  if (!c->live(seq)) return c->fail(LKV_EINVAL, "sequence %d is not live", seq);
  if (layer < 0 || layer >= c->cfg.n_layers || loop < 0 || loop >= c->cfg.n_loops)
    return c->fail(LKV_EINVAL, "cell (%d, %d) out of range", layer, loop);
  const int8_t kind = c->plan[(size_t)layer * c->cfg.n_loops + loop];
  if (kind == LKV_CELL_SHARED) return c->fail(LKV_EINVAL, "cell (%d, %d) is shared and stores no pages", layer, loop);
  if (page0 < 0 || n_pages < 1 || page0 + n_pages > c->max_code_pages)
    return c->fail(LKV_EINVAL, "code pages [%d, %d) outside [0, %d)", page0, page0 + n_pages, c->max_code_pages);
  *T = &c->ctab(layer, loop);
  *fl = kind == LKV_CELL_INT2 ? &c->codes2 : &c->codes4;
  *cpb = kind == LKV_CELL_INT2 ? c->code2_bytes : c->code4_bytes;
  *arena = (uint8_t*)(kind == LKV_CELL_INT2 ? c->ar.codes2 : c->ar.codes4);
  *bits = kind == LKV_CELL_INT2 ? 2 : 4;
  return LKV_OK;
}

// Hand out the pages [page0, page0 + n_pages) of a cell that are not resident yet.
static lkv_status claim_code_pages(lkv_cache* c, Table& T, FreeList& fl, int32_t seq, int32_t page0,
                                   int32_t n_pages) {
  int64_t need = 0;
  for (int p = page0; p < page0 + n_pages; ++p)
    if (T.owner[(size_t)seq * T.ring + p] != p) ++need;
  if (need > fl.available())
    return c->fail(LKV_ENOMEM, "need %lld code pages, %lld free", (long long)need, (long long)fl.available());
  for (int p = page0; p < page0 + n_pages; ++p) {
    const size_t i = (size_t)seq * T.ring + p;
    if (T.owner[i] != p) {
      T.phys[i] = fl.pop();
      T.owner[i] = p;
      T.dirty[(size_t)seq] = 1;
    }
  }
  return LKV_OK;
}

lkv_status lkv_append_coded(lkv_cache* c, int32_t seq, int32_t layer, int32_t loop, int32_t page0, int32_t n_pages,
                            const void* k_codes, const void* k_meta, const void* v_codes, const void* v_meta,
                            void* stream) {
  if (!c) return LKV_EINVAL;
  Table* T;
  FreeList* fl;
  uint8_t* arena;
  uint64_t cpb;
  int bits;
  lkv_status st = code_cell(c, seq, layer, loop, page0, n_pages, &T, &fl, &arena, &cpb, &bits);
  if (st != LKV_OK) return st;
  if (!k_codes || !k_meta || !v_codes || !v_meta) return c->fail(LKV_EINVAL, "NULL code buffer");
  if ((st = claim_code_pages(c, *T, *fl, seq, page0, n_pages)) != LKV_OK) return st;
  T->hi[(size_t)seq] = std::max(T->hi[(size_t)seq], (page0 + n_pages) * kCodePage);
  const int hkv = c->cfg.n_heads_kv, d = c->cfg.head_dim;
  hipStream_t s = (hipStream_t)stream;
  for (int q0 = page0; q0 < page0 + n_pages; q0 += 64) {
    PackParams P{};
    P.arena = arena;
    P.page_bytes = cpb;
    const int64_t k = q0 - page0;
    P.k_codes = (const uint8_t*)k_codes + k * kCodePage * hkv * d;
    P.k_meta = (const uint16_t*)((const uint8_t*)k_meta + k * hkv * d * 4);
    P.v_codes = (const uint8_t*)v_codes + k * kCodePage * hkv * d;
    P.v_meta = (const uint16_t*)((const uint8_t*)v_meta + k * kCodePage * hkv * (d / 32) * 4);
    P.hkv = hkv;
    P.bits = bits;
    P.n_pages = std::min(64, page0 + n_pages - q0);
    for (int x = 0; x < P.n_pages; ++x) P.phys[x] = T->phys[(size_t)seq * T->ring + q0 + x];
    hipError_t e = launch_pack_codes(P, d, s);
    if (e != hipSuccess) return hip_fail(c, e, "pack kernel");
  }
  return LKV_OK;
}

lkv_status lkv_encode_pages(lkv_cache* c, int32_t seq, int32_t layer, int32_t loop, int32_t page0, int32_t n_pages,
                            int32_t n_valid_last, const void* k, const void* v, void* stream) {
  if (!c) return LKV_EINVAL;
  Table* T;
  FreeList* fl;
  uint8_t* arena;
  uint64_t cpb;
  int bits;
  lkv_status st = code_cell(c, seq, layer, loop, page0, n_pages, &T, &fl, &arena, &cpb, &bits);
  if (st != LKV_OK) return st;
  if (!k || !v) return c->fail(LKV_EINVAL, "k and v must not be NULL");
  if (n_valid_last < 1 || n_valid_last > kCodePage)
    return c->fail(LKV_EINVAL, "n_valid_last %d outside [1, %d]", n_valid_last, kCodePage);
  if ((st = claim_code_pages(c, *T, *fl, seq, page0, n_pages)) != LKV_OK) return st;
  T->hi[(size_t)seq] = std::max(T->hi[(size_t)seq], (page0 + n_pages - 1) * kCodePage + n_valid_last);
  const int hkv = c->cfg.n_heads_kv, d = c->cfg.head_dim;
  hipStream_t s = (hipStream_t)stream;
  for (int q0 = page0; q0 < page0 + n_pages; q0 += 64) {
    EncodeParams P{};
    P.arena = arena;
    P.page_bytes = cpb;
    const int64_t off = (int64_t)(q0 - page0) * kCodePage * hkv * d;
    P.k = (const uint16_t*)k + off;
    P.v = (const uint16_t*)v + off;
    P.hkv = hkv;
    P.bits = bits;
    P.n_pages = std::min(64, page0 + n_pages - q0);
    P.n_valid_last = q0 + P.n_pages == page0 + n_pages ? n_valid_last : kCodePage;
    for (int x = 0; x < P.n_pages; ++x) P.phys[x] = T->phys[(size_t)seq * T->ring + q0 + x];
    hipError_t e = launch_encode_pages(P, d, s);
    if (e != hipSuccess) return hip_fail(c, e, "encode kernel");
  }
  return LKV_OK;
}

lkv_status lkv_read_coded(lkv_cache* c, int32_t seq, int32_t layer, int32_t loop, int32_t page0, int32_t n_pages,
                          void* k_codes, void* k_meta, void* v_codes, void* v_meta, void* stream) {
  if (!c) return LKV_EINVAL;
  Table* T;
  FreeList* fl;
  uint8_t* arena;
  uint64_t cpb;
  int bits;
  lkv_status st = code_cell(c, seq, layer, loop, page0, n_pages, &T, &fl, &arena, &cpb, &bits);
  if (st != LKV_OK) return st;
  if (!k_codes || !k_meta || !v_codes || !v_meta) return c->fail(LKV_EINVAL, "NULL code buffer");
  for (int p = page0; p < page0 + n_pages; ++p)
    if (T->owner[(size_t)seq * T->ring + p] != p)
      return c->fail(LKV_ESTATE, "code page %d of cell (%d, %d) is not resident", p, layer, loop);
  const int hkv = c->cfg.n_heads_kv, d = c->cfg.head_dim;
  hipStream_t s = (hipStream_t)stream;
  for (int q0 = page0; q0 < page0 + n_pages; q0 += 64) {
    PackParams P{};
    P.arena = arena;
    P.page_bytes = cpb;
    P.hkv = hkv;
    P.bits = bits;
    P.n_pages = std::min(64, page0 + n_pages - q0);
    for (int x = 0; x < P.n_pages; ++x) P.phys[x] = T->phys[(size_t)seq * T->ring + q0 + x];
    const int64_t k = q0 - page0;
    hipError_t e = launch_read_codes(P, d, (uint8_t*)k_codes + k * kCodePage * hkv * d,
                                     (uint8_t*)k_meta + k * hkv * d * 4, (uint8_t*)v_codes + k * kCodePage * hkv * d,
                                     (uint8_t*)v_meta + k * kCodePage * hkv * (d / 32) * 4, s);
    if (e != hipSuccess) return hip_fail(c, e, "read kernel");
  }
  return LKV_OK;
}

}  // extern "C"

namespace {

struct RowPlan {
  int32_t slot, n_cached, own_lo, deep_hi;
};

// Pages a plain-cache call reads for one sequence: the own plane for positions
// [own_lo, n_cached), the deepest plane for [0, deep_hi).
lkv_status plan_rows(lkv_cache* c, const lkv_attend_args* a, int window, bool ripe, std::vector<RowPlan>* rows) {
  rows->clear();
  const int R = c->cfg.n_loops;
  const Table& To = c->tab(a->layer, a->loop);
  const Table& Td = c->tab(a->layer, R - 1);
  for (int b = 0; b < a->n_seqs; ++b) {
    const int32_t s = a->seq_ids[b];
    if (!c->live(s)) return c->fail(LKV_EINVAL, "seq_ids[%d] = %d is not live", b, s);
    const int32_t n = c->seqs[(size_t)s].len;
    int32_t t_first, t_last, t0;
    if (a->mode == LKV_MODE_DRAFT) {
      t0 = n;
      t_first = t_last = n + a->draft_len - 1;
    } else {
      if (n < a->q_len) return c->fail(LKV_ESTATE, "seq %d has %d positions, fewer than q_len %d", s, n, a->q_len);
      t0 = n - a->q_len;
      t_first = t0;
      t_last = n - 1;
    }
    RowPlan rp{s, n, 0, 0};
    if (ripe) {
      rp.own_lo = std::max(0, std::min(t0, t_first - window));
      rp.deep_hi = std::max(0, std::min(t0, t_last - window));
    }
    if (rp.own_lo < n) {
      if (To.hi[(size_t)s] < n)
        return c->fail(LKV_ESTATE, "seq %d: plane %d of layer %d holds positions below %d, needs %d", s, a->loop,
                       a->layer, To.hi[(size_t)s], n);
      for (int p = rp.own_lo / kPage; p <= (n - 1) / kPage; ++p) {
        const size_t i = (size_t)s * To.ring + (size_t)(p % To.ring);
        if (To.owner[i] != p)
          return c->fail(LKV_ESTATE, "seq %d: page %d of plane %d (layer %d) is not resident", s, p, a->loop,
                         a->layer);
      }
    }
    if (rp.deep_hi > 0) {
      if (Td.hi[(size_t)s] < rp.deep_hi)
        return c->fail(LKV_ESTATE, "seq %d: deepest plane of layer %d holds positions below %d, needs %d", s,
                       a->layer, Td.hi[(size_t)s], rp.deep_hi);
      for (int p = 0; p <= (rp.deep_hi - 1) / kPage; ++p)
        if (Td.owner[(size_t)s * Td.ring + p] != p)
          return c->fail(LKV_ESTATE, "seq %d: page %d of the deepest plane (layer %d) is not resident", s, p,
                         a->layer);
    }
    rows->push_back(rp);
  }
  return LKV_OK;
}

lkv_status upload(lkv_cache* c, Table& T, const std::vector<int32_t>& seq_slots, hipStream_t s) {
  for (int32_t q : seq_slots) {
    if (!T.dirty[(size_t)q]) continue;
    const size_t off = T.dev_off + (size_t)q * T.ring * 4;
    hipError_t e = launch_table_write((int32_t*)((uint8_t*)c->ar.meta + off), T.phys.data() + (size_t)q * T.ring,
                                      T.ring, s);
    if (e != hipSuccess) return hip_fail(c, e, "table upload");
    T.dirty[(size_t)q] = 0;
  }
  return LKV_OK;
}

// Timing events of one chunk of an attend call: the caller's begin event is stamped by
// the first chunk's attention kernel, the end event by the last chunk's (the launch
// itself stamps them, so no marker packets are added to the stream).
LaunchEvents launch_events(const lkv_attend_args* a, bool first, bool last) {
  LaunchEvents ev;
  if (first) ev.start = (hipEvent_t)a->ev_begin;
  if (last) ev.stop = (hipEvent_t)a->ev_end;
  return ev;
}

// Workgroups an automatic split count aims at: eight per CU of the 256-CU MI355X, and two
// per CU for grouped-query decode.
constexpr int kTargetWgs = 2048;
constexpr int kGqaTargetWgs = 512;

// Splits of a plain-cache call: enough workgroups to fill the chip.  Decode and draft
// workgroups serve all query heads of one KV head; verify workgroups the query heads of
// one KV head when the block's rows fit one or two 16-column tiles, else one query head.
// Grouped-query decode aims at two workgroups per CU rather than eight: its kernel time
// hardly depends on the split count (measured on MI355X), and a call without splits
// skips the merge kernel.
int auto_splits(const lkv_cache* c, int n_seqs, int mode, int q_len, int max_pages) {
  const int hq = c->cfg.n_heads_q, hkv = c->cfg.n_heads_kv;
  const int rows =
      n_seqs * (mode == LKV_MODE_VERIFY ? hq / verify_heads_per_wg(hq, hkv, std::max(1, q_len), c->cfg.head_dim) : hkv);
  const bool gqa = mode == LKV_MODE_DECODE && hq > hkv;
  const int target = gqa ? kGqaTargetWgs : kTargetWgs;
  int s = (target + rows - 1) / rows;
  s = std::min(s, std::max(1, max_pages / 8));
  return std::max(1, std::min(s, 64));
}

// Far splits of a quantised-cell call, at most one per code page and at most 64.  The far
// loops are software-pipelined at five waves per SIMD (a wave keeps the next page's loads in
// flight while it computes the current one; INT4: the next page's scores while the current
// page's lo rows are in flight), which pays off over long runs of pages: a call takes as many
// splits as keep the whole grid, near blocks included, resident at once (five 4-wave
// workgroups per CU on the 256 CUs; one split more and the last far blocks start a whole
// block late; measured on MI355X, for the running rule too, whose far blocks meet at a
// barrier once per round of pages).
constexpr int kCellPipelinedWgs = 5 * 256;

int cell_splits(const lkv_cache* c, int n_seqs, int split_k, int max_code_pages) {
  const int rows = n_seqs * c->cfg.n_heads_q;
  const int S = split_k > 0 ? split_k : std::max(1, std::min(64, kCellPipelinedWgs / rows - 1));
  return std::min(S, std::max(1, max_code_pages));
}

}  // namespace

extern "C" {

lkv_status lkv_workspace_bytes(const lkv_cache* c, const lkv_attend_args* a, size_t* bytes) {
  if (!c || !a || !bytes) return LKV_EINVAL;
  int max_pages = 0, max_cp = 0;
  for (int b = 0; b < a->n_seqs && a->seq_ids; ++b) {
    const int32_t s = a->seq_ids[b];
    if (s < 0 || s >= c->cfg.max_seqs) continue;
    const int L = c->seqs[(size_t)s].len;
    max_pages = std::max(max_pages, (L + kPage - 1) / kPage);
    max_cp = std::max(max_cp, (std::max(0, L - c->cfg.sink - c->cfg.tail) + kCodePage - 1) / kCodePage);
  }
  const int S = c->cfg.quant ? cell_splits(c, a->n_seqs, a->split_k, max_cp)
                             : (a->split_k > 0 ? a->split_k : auto_splits(c, a->n_seqs, a->mode, a->q_len, max_pages));
  const int parts = c->cfg.quant ? S + 1 : S;
  if (parts <= 1) {
    *bytes = 0;
    return LKV_OK;
  }
  const int q_len = std::max(1, a->q_len);
  *bytes = (size_t)a->n_seqs * q_len * c->cfg.n_heads_q * parts * (c->cfg.head_dim + 1) * 4;
  return LKV_OK;
}

static lkv_status attend_cell(lkv_cache* c, const lkv_attend_args* a, hipStream_t s);

lkv_status lkv_attend(lkv_cache* c, const lkv_attend_args* a, void* stream) {
  if (!c) return LKV_EINVAL;
  if (!a) return c->fail(LKV_EINVAL, "args is NULL");
  const auto& cfg = c->cfg;
  if (a->layer < 0 || a->layer >= cfg.n_layers || a->loop < 0 || a->loop >= cfg.n_loops)
    return c->fail(LKV_EINVAL, "(layer %d, loop %d) out of range", a->layer, a->loop);
  if (a->n_seqs < 1 || a->n_seqs > cfg.max_seqs || !a->seq_ids)
    return c->fail(LKV_EINVAL, "n_seqs %d outside [1, %d] or seq_ids NULL", a->n_seqs, cfg.max_seqs);
  if (!a->q || !a->out) return c->fail(LKV_EINVAL, "q and out must not be NULL");
  if (a->mode != LKV_MODE_DECODE && a->mode != LKV_MODE_VERIFY && a->mode != LKV_MODE_DRAFT)
    return c->fail(LKV_EINVAL, "mode %d", a->mode);
  if (a->mode == LKV_MODE_VERIFY ? (a->q_len < 1 || a->q_len > cfg.max_block) : a->q_len != 1)
    return c->fail(LKV_EINVAL, "q_len %d does not fit mode %d (max_block %d)", a->q_len, a->mode, cfg.max_block);
  if (a->mode == LKV_MODE_DRAFT) {
    if (a->draft_len < 1 || a->draft_len > cfg.max_block || !a->draft_k || !a->draft_v)
      return c->fail(LKV_EINVAL, "draft needs 1 <= draft_len <= %d and draft_k/draft_v", cfg.max_block);
  }
  if (a->split_k < 0 || a->split_k > 64) return c->fail(LKV_EINVAL, "split_k %d outside [0, 64]", a->split_k);
  if (a->index_trace && a->trace_len < 1) return c->fail(LKV_EINVAL, "trace_len must be >= 1");
  if (a->window < -1) return c->fail(LKV_EINVAL, "window %d", a->window);
  if (a->v_rule != LKV_VRULE_FIXED && a->v_rule != LKV_VRULE_RUNNING)
    return c->fail(LKV_EINVAL, "v_rule %d", a->v_rule);
  if (a->v_rule == LKV_VRULE_RUNNING && !(a->v_tau >= 0.f)) return c->fail(LKV_EINVAL, "v_tau must be >= 0");
  if (a->kernel != LKV_KERNEL_AUTO && a->kernel != LKV_KERNEL_VALU) return c->fail(LKV_EINVAL, "kernel %d", a->kernel);
  if (a->waves < 0) return c->fail(LKV_EINVAL, "waves %d", a->waves);
  hipStream_t s = (hipStream_t)stream;
  if (cfg.quant) return attend_cell(c, a, s);

  // q = 1 decode of a grouped-query cache runs on the MFMA kernel (its G query heads are
  // G columns of one tile); multi-head decode and the draft on the VALU decode kernel.
  const int group = cfg.n_heads_q / cfg.n_heads_kv;
  const bool gqa = a->mode == LKV_MODE_DECODE && (group == 2 || group == 4 || group == 8) &&
                   a->kernel == LKV_KERNEL_AUTO;
  const int window = a->window < 0 ? cfg.window : a->window;
  const int R = cfg.n_loops;
  const bool ripe = cfg.policy == LKV_POLICY_RIPE && a->loop != R - 1;
  std::vector<RowPlan> rows;
  lkv_status st = plan_rows(c, a, window, ripe, &rows);
  if (st != LKV_OK) return st;
  int max_pages = 0;
  for (const auto& r : rows) max_pages = std::max(max_pages, (r.n_cached + kPage - 1) / kPage);
  const int S = a->split_k > 0 ? a->split_k : auto_splits(c, a->n_seqs, a->mode, a->q_len, max_pages);
  // Waves per workgroup (defaults measured best on MI355X): 2 for verify tiles, 4 for
  // grouped-query rows (and the grouped VALU kernel, whose registers grow with G), and for
  // multi-head q = 1 rows 8, except 2 when the grid has 768-1024 workgroups: there the 8-wave
  // grid is about one generation of resident waves (seven per SIMD) and 2-wave workgroups, at
  // 1.5-2 waves per SIMD with twice the pages per wave, measured 1-8% faster (Huginn shape at
  // 14, 16 and 18 sequences: 52.4 -> 48.1, 57.4 -> 54.8, 61.8 -> 61.0 us); below that band
  // they leave SIMDs idle (12 sequences: 44.3 -> 45.1 us), above it 8 waves stay ahead.
  const int64_t wgs = (int64_t)a->n_seqs * cfg.n_heads_kv * S;
  const int waves = a->waves > 0 ? a->waves
                    : a->mode == LKV_MODE_VERIFY ? 2
                    : gqa                        ? 4
                    : group != 1                 ? 4
                    : (wgs >= 768 && wgs <= 1024) ? 2
                                                  : 8;
  const bool waves_ok = a->mode == LKV_MODE_VERIFY ? (waves == 1 || waves == 2 || waves == 4)
                        : gqa                      ? (waves == 1 || waves == 2 || waves == 4)
                                                   : (waves == 2 || waves == 4 || waves == 8);
  if (!waves_ok) return c->fail(LKV_EINVAL, "waves %d is not built for this kernel", waves);
  const int D = cfg.head_dim, hq = cfg.n_heads_q, es = elem_bytes(cfg);
  const size_t ws_need = S > 1 ? (size_t)a->n_seqs * a->q_len * hq * S * (D + 1) * 4 : 0;
  if (ws_need > 0 && (!a->workspace || a->workspace_bytes < ws_need))
    return c->fail(LKV_ENOMEM, "workspace of %zu bytes needed for %d splits", ws_need, S);

  Table& To = c->tab(a->layer, a->loop);
  Table& Td = c->tab(a->layer, R - 1);
  std::vector<int32_t> slots;
  for (const auto& r : rows) slots.push_back(r.slot);
  if ((st = upload(c, To, slots, s)) != LKV_OK) return st;
  if (&To != &Td && (st = upload(c, Td, slots, s)) != LKV_OK) return st;

  if (a->index_trace) {
    hipError_t e = launch_fill(a->index_trace, (uint64_t)a->n_seqs * a->q_len * a->trace_len * 8, 0xFFFFFFFFu, s);
    if (e != hipSuccess) return hip_fail(c, e, "trace clear");
  }
  const int64_t qrow = (int64_t)a->q_len * hq * D;
  for (int b0 = 0; b0 < a->n_seqs; b0 += kMaxRows) {
    const int nb = std::min(kMaxRows, a->n_seqs - b0);
    PlainParams P{};
    P.pool = (const uint8_t*)c->ar.pages;
    P.page_bytes = c->page_bytes;
    P.tab_own = (const int32_t*)((const uint8_t*)c->ar.meta + (ripe ? To.dev_off : To.dev_off));
    P.tab_deep = (const int32_t*)((const uint8_t*)c->ar.meta + Td.dev_off);
    P.ring_own = To.ring;
    P.ring_deep = Td.ring;
    P.q = (const uint8_t*)a->q + b0 * qrow * es;
    P.out = (uint8_t*)a->out + b0 * qrow * es;
    P.lse = a->lse ? a->lse + (int64_t)b0 * a->q_len * hq : nullptr;
    P.ws = S > 1 ? (float*)a->workspace + (int64_t)b0 * a->q_len * hq * S * (D + 1) : nullptr;
    if (a->mode == LKV_MODE_DRAFT) {
      const int64_t drow = (int64_t)a->draft_len * cfg.n_heads_kv * D * es;
      P.draft_k = (const uint8_t*)a->draft_k + b0 * drow;
      P.draft_v = (const uint8_t*)a->draft_v + b0 * drow;
      P.draft_len = a->draft_len;
    }
    P.trace = a->index_trace ? a->index_trace + (int64_t)b0 * a->q_len * a->trace_len * 2 : nullptr;
    P.trace_len = a->trace_len;
    P.n_rows = nb;
    P.q_len = a->q_len;
    P.hq = hq;
    P.hkv = cfg.n_heads_kv;
    P.window = window;
    P.ripe = ripe ? 1 : 0;
    P.loop = a->loop;
    P.deepest = R - 1;
    P.n_splits = S;
    P.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
    for (int b = 0; b < nb; ++b) {
      P.slot[b] = rows[(size_t)(b0 + b)].slot;
      P.len[b] = rows[(size_t)(b0 + b)].n_cached;
    }
    const bool tr = a->index_trace != nullptr;
    const LaunchEvents ev = launch_events(a, b0 == 0, b0 + nb >= a->n_seqs);
    hipError_t e = a->mode == LKV_MODE_VERIFY ? launch_verify(P, cfg.kv_dtype, D, waves, tr, s, ev)
                   : gqa                     ? launch_gqa_decode(P, cfg.kv_dtype, D, waves, tr, s, ev)
                                             : launch_decode(P, cfg.kv_dtype, D, waves, tr, s, ev);
    if (e != hipSuccess) return hip_fail(c, e, "attention kernel");
    if (S > 1) {
      MergeParams M{};
      M.ws = P.ws;
      M.out = P.out;
      M.lse = P.lse;
      M.n_rows = nb * a->q_len * hq;
      M.n_parts = S;
      e = launch_merge(M, cfg.kv_dtype, D, s);
      if (e != hipSuccess) return hip_fail(c, e, "merge kernel");
    }
  }
  return LKV_OK;
}

static lkv_status attend_cell(lkv_cache* c, const lkv_attend_args* a, hipStream_t s) {
  const auto& cfg = c->cfg;
  if (a->mode != LKV_MODE_DECODE) return c->fail(LKV_EUNSUPPORTED, "quantised cells serve decode only");
  const int waves = a->waves > 0 ? a->waves : 4;
  if (waves != 2 && waves != 4) return c->fail(LKV_EINVAL, "waves %d is not built for the cell kernel", waves);
  if (!c->plan_set) return c->fail(LKV_ESTATE, "lkv_set_plan first");
  const int R = cfg.n_loops;
  const int8_t kind = c->plan[(size_t)a->layer * R + a->loop];
  const int src_loop = kind == LKV_CELL_SHARED ? R - 1 : a->loop;
  const int8_t src_kind = c->plan[(size_t)a->layer * R + src_loop];
  const int bits = src_kind == LKV_CELL_INT2 ? 2 : 4;
  Table& Tn = c->tab(a->layer, a->loop);
  Table& Tc = c->ctab(a->layer, src_loop);
  std::vector<int32_t> slots;
  int max_far = 0;
  for (int b = 0; b < a->n_seqs; ++b) {
    const int32_t sq = a->seq_ids[b];
    if (!c->live(sq)) return c->fail(LKV_EINVAL, "seq_ids[%d] = %d is not live", b, sq);
    const int32_t L = c->seqs[(size_t)sq].len;
    if (L < cfg.sink + cfg.tail + 1)
      return c->fail(LKV_ESTATE, "seq %d: length %d below sink + tail + 1 = %d", sq, L, cfg.sink + cfg.tail + 1);
    const int n_far = L - cfg.sink - cfg.tail;
    max_far = std::max(max_far, n_far);
    const int n_cp = (n_far + kCodePage - 1) / kCodePage;
    if (n_cp > c->max_code_pages) return c->fail(LKV_ESTATE, "seq %d: far history longer than max_len", sq);
    if (Tc.hi[(size_t)sq] < n_far)
      return c->fail(LKV_ESTATE, "seq %d: cell (%d, %d) holds %d far positions as codes, the call needs %d "
                     "(lkv_window_exit encodes the positions that left the tail)", sq, a->layer, src_loop,
                     Tc.hi[(size_t)sq], n_far);
    for (int p = 0; p < n_cp; ++p)
      if (Tc.owner[(size_t)sq * Tc.ring + p] != p)
        return c->fail(LKV_ESTATE, "seq %d: code page %d of cell (%d, %d) is not resident", sq, p, a->layer, src_loop);
    // near pages: sink [0, sink) and tail [L - tail, L)
    auto need_page = [&](int p) { return Tn.owner[(size_t)sq * Tn.ring + p] == p; };
    for (int p = 0; p <= (cfg.sink - 1) / kPage; ++p)
      if (!need_page(p)) return c->fail(LKV_ESTATE, "seq %d: sink page %d of loop %d is not resident", sq, p, a->loop);
    if (cfg.tail > 0)
      for (int p = (L - cfg.tail) / kPage; p <= (L - 1) / kPage; ++p)
        if (!need_page(p))
          return c->fail(LKV_ESTATE, "seq %d: tail page %d of loop %d is not resident", sq, p, a->loop);
    slots.push_back(sq);
  }
  const int D = cfg.head_dim, hq = cfg.n_heads_q;
  const int max_cp = (max_far + kCodePage - 1) / kCodePage;
  const int S = cell_splits(c, a->n_seqs, a->split_k, max_cp);
  const size_t ws_need = (size_t)a->n_seqs * hq * (S + 1) * (D + 1) * 4;
  if (!a->workspace || a->workspace_bytes < ws_need)
    return c->fail(LKV_ENOMEM, "workspace of %zu bytes needed", ws_need);
  lkv_status st;
  if ((st = upload(c, Tn, slots, s)) != LKV_OK) return st;
  if ((st = upload(c, Tc, slots, s)) != LKV_OK) return st;
  const int mask_words = (max_far + 31) / 32;
  if (a->mask_trace) {
    hipError_t e = launch_fill(a->mask_trace, (uint64_t)a->n_seqs * hq * mask_words * 4, 0u, s);
    if (e != hipSuccess) return hip_fail(c, e, "mask clear");
  }
  for (int b0 = 0; b0 < a->n_seqs; b0 += kMaxRows) {
    const int nb = std::min(kMaxRows, a->n_seqs - b0);
    CellParams P{};
    P.pool = (const uint8_t*)c->ar.pages;
    P.page_bytes = c->page_bytes;
    P.tab_near = (const int32_t*)((const uint8_t*)c->ar.meta + Tn.dev_off);
    P.ring_near = Tn.ring;
    P.codes = (const uint8_t*)(bits == 2 ? c->ar.codes2 : c->ar.codes4);
    P.code_page_bytes = bits == 2 ? c->code2_bytes : c->code4_bytes;
    P.tab_code = (const int32_t*)((const uint8_t*)c->ar.meta + Tc.dev_off);
    P.code_ring = Tc.ring;
    P.bits = bits;
    P.masked = bits == 4 ? 1 : 0;
    P.thr_offset = a->v_thresh_offset;
    P.rule = a->v_rule;
    P.v_tau = a->v_tau;
    P.q = (const uint8_t*)a->q + (int64_t)b0 * hq * D * 2;
    P.out = (uint8_t*)a->out + (int64_t)b0 * hq * D * 2;
    P.lse = a->lse ? a->lse + (int64_t)b0 * hq : nullptr;
    P.ws = (float*)a->workspace + (int64_t)b0 * hq * (S + 1) * (D + 1);
    P.mask_trace = a->mask_trace ? a->mask_trace + (int64_t)b0 * hq * mask_words : nullptr;
    P.mask_words = mask_words;
    P.n_rows = nb;
    P.hq = hq;
    P.hkv = cfg.n_heads_kv;
    P.sink = cfg.sink;
    P.tail = cfg.tail;
    P.n_splits = S;
    P.scale = (float)(1.0 / std::sqrt((double)D));
    P.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
    for (int b = 0; b < nb; ++b) {
      P.slot[b] = slots[(size_t)(b0 + b)];
      P.len[b] = c->seqs[(size_t)slots[(size_t)(b0 + b)]].len;
    }
    hipError_t e = launch_cell(P, D, waves, s, launch_events(a, b0 == 0, b0 + nb >= a->n_seqs));
    if (e != hipSuccess) return hip_fail(c, e, "cell kernel");
    MergeParams M{};
    M.ws = P.ws;
    M.out = P.out;
    M.lse = P.lse;
    M.n_rows = nb * hq;
    M.n_parts = S + 1;
    e = launch_merge(M, LKV_DTYPE_BF16, D, s);
    if (e != hipSuccess) return hip_fail(c, e, "merge kernel");
  }
  return LKV_OK;
}

lkv_status lkv_mem_stats(const lkv_cache* c, lkv_mem_info* out) {
  if (!c || !out) return LKV_EINVAL;
  const auto& cfg = c->cfg;
  const int64_t b = 2ll * cfg.n_heads_kv * cfg.head_dim * elem_bytes(cfg);  // bytes per layer per token
  int64_t logical = 0;
  for (int s = 0; s < cfg.max_seqs; ++s) {
    const auto& S = c->seqs[(size_t)s];
    if (!S.live) continue;
    const int64_t L = S.len;
    if (!cfg.quant) {
      if (cfg.policy == LKV_POLICY_FULL) logical += b * L * cfg.n_layers * cfg.n_loops;
      else logical += b * cfg.n_layers * (L + (int64_t)(cfg.n_loops - 1) * std::min<int64_t>(cfg.window, L));
    } else {
      const int64_t near = std::min<int64_t>(L, cfg.sink) + std::min<int64_t>(cfg.tail, std::max<int64_t>(0, L - cfg.sink));
      const int64_t far = std::max<int64_t>(0, L - cfg.sink - cfg.tail);
      for (int l = 0; l < cfg.n_layers; ++l)
        for (int r = 0; r < cfg.n_loops; ++r) {
          const int8_t k = c->plan[(size_t)l * cfg.n_loops + r];
          logical += b * near;
          if (k == LKV_CELL_INT4) logical += far * 2ll * cfg.n_heads_kv * cfg.head_dim * 5 / 8;
          if (k == LKV_CELL_INT2) logical += far * 2ll * cfg.n_heads_kv * cfg.head_dim * 3 / 8;
        }
    }
  }
  out->logical_bytes = logical;
  out->pages_in_use = c->pages.in_use();
  out->pages_total = c->pages.total;
  out->code4_in_use = c->codes4.in_use();
  out->code4_total = c->codes4.total;
  out->code2_in_use = c->codes2.in_use();
  out->code2_total = c->codes2.total;
  return LKV_OK;
}

lkv_status lkv_debug_resolve(const lkv_cache* c, int32_t seq, int32_t layer, int32_t loop, int32_t t, int32_t t0,
                             int32_t j, int32_t window, int32_t* plane, int32_t* phys_page, int32_t* slot) {
  if (!c || !plane || !phys_page || !slot) return LKV_EINVAL;
  if (!c->live(seq) || layer < 0 || layer >= c->cfg.n_layers || loop < 0 || loop >= c->cfg.n_loops || j < 0 ||
      j > t || t0 > t || j >= c->cfg.max_len)
    return LKV_EINVAL;
  const int W = window < 0 ? c->cfg.window : window;
  const int R = c->cfg.n_loops;
  int p = loop;
  if (c->cfg.policy == LKV_POLICY_RIPE && !c->cfg.quant && j < t0 && t - j > W) p = R - 1;
  const Table& T = c->tab(layer, p);
  const int lp = j / kPage;
  const size_t i = (size_t)seq * T.ring + (size_t)(lp % T.ring);
  *plane = p;
  *phys_page = T.owner[i] == lp ? T.phys[i] : -1;
  *slot = j % kPage;
  return LKV_OK;
}

lkv_status lkv_seq_info(const lkv_cache* c, int32_t seq, int32_t* len, int32_t* committed) {
  if (!c || !len || !committed) return LKV_EINVAL;
  if (!c->live(seq)) return LKV_EINVAL;
  *len = c->seqs[(size_t)seq].len;
  *committed = c->seqs[(size_t)seq].committed;
  return LKV_OK;
}

lkv_status lkv_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* ev_begin, void* ev_end,
                          void* stream) {
  if (!buf || !sink) return LKV_EINVAL;
  if (bytes < LKV_PROBE_CHUNK || bytes % LKV_PROBE_CHUNK != 0 || bytes / LKV_PROBE_CHUNK > 0x7FFFFFFFull)
    return LKV_EINVAL;
  LaunchEvents ev;
  ev.start = (hipEvent_t)ev_begin;
  ev.stop = (hipEvent_t)ev_end;
  return launch_probe_read(buf, bytes, sink, (hipStream_t)stream, ev) == hipSuccess ? LKV_OK : LKV_EDEVICE;
}

}  // extern "C"

// ----------------------------------------------------------------------------- window exit of quantised caches

extern "C" lkv_status lkv_window_exit(lkv_cache* c, int32_t seq, void* stream) {
  if (!c) return LKV_EINVAL;
  const auto& cfg = c->cfg;
  if (!cfg.quant) return c->fail(LKV_ESTATE, "the cache has no quantised cells");
  if (!c->plan_set) return c->fail(LKV_ESTATE, "lkv_set_plan first");
  if (!c->live(seq)) return c->fail(LKV_EINVAL, "sequence %d is not live", seq);
  const int R = cfg.n_loops, nl = cfg.n_layers;
  const int32_t L = c->seqs[(size_t)seq].len;
  const int32_t fe = std::max(0, L - cfg.tail - cfg.sink);  // far positions that left the tail
  if ((fe + kCodePage - 1) / kCodePage > c->max_code_pages)
    return c->fail(LKV_ESTATE, "far history of seq %d longer than max_len allows", seq);
  // Phase 1 (host checks, nothing changes): the positions to encode are resident in each
  // cell's exact plane, and the pools hold the code pages that are needed.
  int64_t need4 = 0, need2 = 0;
  for (int l = 0; l < nl; ++l)
    for (int r = 0; r < R; ++r) {
      const int8_t kind = c->plan[(size_t)l * R + r];
      if (kind == LKV_CELL_SHARED) continue;
      const Table& Tc = c->ctab(l, r);
      const int32_t done = Tc.hi[(size_t)seq];
      if (fe <= done) continue;
      const int32_t p0 = done / kCodePage, p1 = (fe - 1) / kCodePage;
      for (int p = p0; p <= p1; ++p)
        if (Tc.owner[(size_t)seq * Tc.ring + p] != p) ++(kind == LKV_CELL_INT2 ? need2 : need4);
      const Table& Tn = c->tab(l, r);
      const int32_t a = cfg.sink + p0 * kCodePage, b = cfg.sink + fe;
      if (Tn.hi[(size_t)seq] < b)
        return c->fail(LKV_ESTATE, "seq %d: plane %d of layer %d holds positions below %d, the exit needs %d", seq, r,
                       l, Tn.hi[(size_t)seq], b);
      for (int pg = a / kPage; pg <= (b - 1) / kPage; ++pg)
        if (Tn.owner[(size_t)seq * Tn.ring + pg] != pg)
          return c->fail(LKV_ESTATE, "seq %d: page %d of plane %d (layer %d) is not resident", seq, pg, r, l);
    }
  if (need4 > c->codes4.available() || need2 > c->codes2.available())
    return c->fail(LKV_ENOMEM, "need %lld INT4 and %lld INT2 code pages, %lld and %lld free", (long long)need4,
                   (long long)need2, (long long)c->codes4.available(), (long long)c->codes2.available());
  // Phase 2: encode every non-shared cell's new far positions from its exact plane (the
  // partial last page is encoded again from all its valid tokens), on the stream.
  hipStream_t s = (hipStream_t)stream;
  const int hkv = cfg.n_heads_kv, d = cfg.head_dim;
  const std::vector<int32_t> one{seq};
  for (int l = 0; l < nl; ++l)
    for (int r = 0; r < R; ++r) {
      const int8_t kind = c->plan[(size_t)l * R + r];
      if (kind == LKV_CELL_SHARED) continue;
      Table& Tc = c->ctab(l, r);
      const int32_t done = Tc.hi[(size_t)seq];
      if (fe <= done) continue;
      FreeList& fl = kind == LKV_CELL_INT2 ? c->codes2 : c->codes4;
      const int32_t p0 = done / kCodePage, p1 = (fe - 1) / kCodePage;
      lkv_status st = claim_code_pages(c, Tc, fl, seq, p0, p1 - p0 + 1);
      if (st != LKV_OK) return st;  // cannot happen after phase 1
      Table& Tn = c->tab(l, r);
      if ((st = upload(c, Tn, one, s)) != LKV_OK) return st;
      for (int q0 = p0; q0 <= p1; q0 += 64) {
        EncodeParams P{};
        P.arena = (uint8_t*)(kind == LKV_CELL_INT2 ? c->ar.codes2 : c->ar.codes4);
        P.page_bytes = kind == LKV_CELL_INT2 ? c->code2_bytes : c->code4_bytes;
        P.pool = (const uint8_t*)c->ar.pages;
        P.plain_page_bytes = c->page_bytes;
        P.tab_plain = (const int32_t*)((const uint8_t*)c->ar.meta + Tn.dev_off) + (size_t)seq * Tn.ring;
        P.pos0 = cfg.sink + q0 * kCodePage;
        P.hkv = hkv;
        P.bits = kind == LKV_CELL_INT2 ? 2 : 4;
        P.n_pages = std::min(64, p1 + 1 - q0);
        P.n_valid_last = q0 + P.n_pages - 1 == p1 ? fe - p1 * kCodePage : kCodePage;
        for (int x = 0; x < P.n_pages; ++x) P.phys[x] = Tc.phys[(size_t)seq * Tc.ring + q0 + x];
        hipError_t e = launch_encode_pages(P, d, s);
        if (e != hipSuccess) return hip_fail(c, e, "encode kernel");
      }
      Tc.hi[(size_t)seq] = fe;
    }
  // Phase 3: release the exact pages no cell reads any more: pages wholly past the sink
  // whose positions all lie in complete code pages (a cell with codes), or that all left
  // the tail (a shared cell, which reads the final loop's codes).  Released pages go back
  // to the pool; device work that writes them again must follow this call's kernels on
  // the stream.
  const int32_t whole = cfg.sink + fe / kCodePage * kCodePage;
  for (int l = 0; l < nl; ++l)
    for (int r = 0; r < R; ++r) {
      const int32_t limit = c->plan[(size_t)l * R + r] == LKV_CELL_SHARED ? cfg.sink + fe : whole;
      Table& Tn = c->tab(l, r);
      for (int e = 0; e < Tn.ring; ++e) {
        const size_t i = (size_t)seq * Tn.ring + e;
        const int32_t o = Tn.owner[i];
        if (o >= 0 && o * kPage >= cfg.sink && (o + 1) * kPage <= limit) {
          c->pages.push(Tn.phys[i]);
          Tn.phys[i] = -1;
          Tn.owner[i] = -1;
          Tn.dirty[(size_t)seq] = 1;
        }
      }
    }
  return LKV_OK;
}

// ----------------------------------------------------------------------------- attend without allocation
//
// lkv_attend_noalloc runs lkv_attend with the split partials in a fixed device array
// instead of a caller workspace, for callers that cannot allocate.  The array is one
// file-scope __device__ object: every GPU the library runs on holds its own copy until
// the process ends, at its own address, which is looked up once per device with
// hipGetSymbolAddress (the array's name in host code is only a host-side stand-in).
// The partials are written in full before they are read, so nothing in it has to start
// at zero; calls that overlap on one device share it and race.
static __device__ __align__(256) uint8_t scratch[LKV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of the scratch array (resolved on first use, with
// the device current).
hipError_t scratch_ptr(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return e;
    if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (prev != device) {
      const hipError_t e2 = hipSetDevice(prev);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}
}  // namespace

extern "C" {

lkv_status lkv_attend_noalloc(lkv_cache* c, const lkv_attend_args* a, void* stream) {
  if (!c) return LKV_EINVAL;
  if (!a) return c->fail(LKV_EINVAL, "args is NULL");
  if (a->workspace || a->workspace_bytes)
    return c->fail(LKV_EINVAL, "lkv_attend_noalloc takes no workspace (its partials live in the library's scratch)");
  if (c->device < 0 || c->device >= kMaxDevices) return c->fail(LKV_EINVAL, "device %d", c->device);
  size_t need = 0;
  lkv_status st = lkv_workspace_bytes(c, a, &need);
  if (st != LKV_OK) return c->fail(st, "workspace size of the call");
  if (need > LKV_NOALLOC_SCRATCH_BYTES)
    return c->fail(LKV_EINVAL, "the call needs %zu bytes of partials, more than the %zu-byte scratch of "
                   "lkv_attend_noalloc (fewer splits or sequences per call, or lkv_attend with a workspace)",
                   need, (size_t)LKV_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  hipError_t e = scratch_ptr(c->device, &ptr);
  if (e != hipSuccess) return hip_fail(c, e, "scratch address (hipGetSymbolAddress)");
  lkv_attend_args b = *a;
  b.workspace = ptr;
  b.workspace_bytes = LKV_NOALLOC_SCRATCH_BYTES;
  return lkv_attend(c, &b, stream);
}

}  // extern "C"
