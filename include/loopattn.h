/*
 * loopattn: loop-aware attention over a looped (recurrent-depth) language
 * model's multi-plane KV cache, for AMD Instinct MI355X (gfx950).
 *
 * A looped model runs a block of core layers R times per token; loop r of each
 * core layer writes its own keys and values, "plane r" ("Prefix Keys and Values
 * Matter Late: RIPE Caching for Self-Speculative Decoding in Looped Language
 * Models", Sec. 2).  At loop r each query token attends to its sequence's keys
 * and values, read from the plane a cache policy names:
 *
 *   FULL  every position reads plane r                       (RIPE page, Sec. 2)
 *   RIPE  plane r if t - j <= W, else the deepest plane R    (RIPE page, Eq. (9))
 *         (W = 0 is the deepest-plane cache; positions of the query's own block
 *          always read plane r, proof of Prop. 1)
 *   cells LoopKV-style quantised (layer, loop) cells: INT4 or INT2 codes for the
 *         history, or a pointer redirection to the final loop's codes; exact
 *         sink and tail ("LoopKV: Loop-Aware KV Cache Compression for Serving
 *         Looped Transformers", Sec. 3.1-3.4).
 *
 * Conventions used by every call:
 *   - loops are 0-based: loop in [0, n_loops), deepest = n_loops - 1;
 *   - a sequence of length L holds positions 0..L-1, including the query (or
 *     the verify block) being attended; q_len rows sit at t0 = L - q_len .. L-1
 *     and row t sees keys j <= t;
 *   - the score scale is 1/sqrt(head_dim); lse outputs are natural logs;
 *   - all device memory is caller-owned (e.g. PyTorch tensors); the library
 *     never allocates device memory;
 *   - `stream` arguments are hipStream_t handles (NULL = the null stream); all
 *     device work is asynchronous on that stream; nothing synchronises;
 *   - every call returns lkv_status; on error the handle is unchanged and stays
 *     usable, and lkv_last_error() describes the failure;
 *   - a handle is bound to one device and is not thread-safe.
 */
#ifndef LOOPATTN_H
#define LOOPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LKV_OK = 0,
  LKV_EINVAL = 1,       /* bad argument: shape, index, range, NULL pointer */
  LKV_ENOMEM = 2,       /* an arena or the page pool is exhausted */
  LKV_ESTATE = 3,       /* cache state does not allow the call (missing plane, gap, dead seq) */
  LKV_EWINDOW = 4,      /* RIPE: a non-deepest plane written outside the window ring */
  LKV_EDEVICE = 5,      /* a HIP call or kernel launch failed */
  LKV_EUNSUPPORTED = 6  /* valid request that this build does not implement */
} lkv_status;

enum { LKV_DTYPE_F32 = 0, LKV_DTYPE_BF16 = 1 };
enum { LKV_POLICY_FULL = 0, LKV_POLICY_RIPE = 1 };
enum { LKV_MODE_DECODE = 0, LKV_MODE_VERIFY = 1, LKV_MODE_DRAFT = 2 };
/* Cell kinds of a quantised cache (LoopKV page, Sec. 3.1-3.2).  BF16 is reserved. */
enum { LKV_CELL_BF16 = 0, LKV_CELL_INT4 = 1, LKV_CELL_INT2 = 2, LKV_CELL_SHARED = 3 };
/* Hot test of a far token in an INT4 or shared cell (which decides whether its V lo
   plane is read; LoopKV page, Sec. 3.3).  FIXED: s_j >= m0 - v_thresh_offset, with m0
   the largest sink score.  RUNNING (the page's own rule, App. E Algorithm 1): the far
   history's 32-token pages are shared out to the call's far splits, split c taking
   pages [floor(c n / S), floor((c + 1) n / S)); a split walks its pages in order and
   token j of page p is hot iff s_j >= max(m, m0) - v_tau ln 2, where m is the largest
   score of the split's pages up to and including p.  Scores are logits in natural
   units (q.k / sqrt(d)); ties are hot. */
enum { LKV_VRULE_FIXED = 0, LKV_VRULE_RUNNING = 1 };
/* Kernel choice of an attend call (lkv_attend_args.kernel).  AUTO: q = 1 decode of a
   grouped-query cache runs on the MFMA tile kernel, everything else on its own kernel.
   VALU: grouped-query decode on the VALU decode kernel instead (the draft step always
   runs there). */
enum { LKV_KERNEL_AUTO = 0, LKV_KERNEL_VALU = 1 };

/* Tokens per plain page and per code page. */
#define LKV_PAGE_TOKENS 16
#define LKV_CODE_PAGE_TOKENS 32

typedef struct {
  int32_t n_layers;     /* core (looped) layers */
  int32_t n_loops;      /* R */
  int32_t n_heads_q;    /* query heads */
  int32_t n_heads_kv;   /* KV heads; n_heads_q % n_heads_kv == 0 */
  int32_t head_dim;     /* 64, 96, 128, or 256 (bf16 caches, plain planes) */
  int32_t page_size;    /* tokens per plain page: must be LKV_PAGE_TOKENS */
  int32_t kv_dtype;     /* LKV_DTYPE_F32 or LKV_DTYPE_BF16 (also the q / out dtype) */
  int32_t policy;       /* LKV_POLICY_FULL or LKV_POLICY_RIPE */
  int32_t window;       /* RIPE window W >= 0 */
  int32_t max_seqs;     /* sequence slots */
  int32_t max_len;      /* longest sequence, positions */
  int32_t max_block;    /* longest verify block (q_len), 1..16 */
  int32_t quant;        /* 0: plain planes; 1: LoopKV-style cells (bf16, FULL) */
  int32_t sink;         /* quant: exact sink positions [0, sink), 1..64 (the page's rule uses 32) */
  int32_t tail;         /* quant: exact tail positions [L - tail, L) */
  int32_t poison;       /* 1: fill pages with NaN when handed out (debug) */
  uint64_t shuffle_seed;/* 0: free pages handed out in address order; else a seeded permutation */
} lkv_config;

/* Caller-owned device arenas.  Sizes come from lkv_sizes(). */
typedef struct {
  void* pages;  size_t pages_bytes;   /* plain pages */
  void* codes4; size_t codes4_bytes;  /* INT4 code pages (quant only) */
  void* codes2; size_t codes2_bytes;  /* INT2 code pages (quant only) */
  void* meta;   size_t meta_bytes;    /* device block tables: exactly lkv_size_info.meta_bytes or more */
} lkv_arenas;

typedef struct {
  size_t page_bytes;       /* one plain page: all KV heads, 16 tokens, K and V */
  size_t code4_page_bytes; /* one INT4 code page: all KV heads, 32 tokens */
  size_t code2_page_bytes; /* one INT2 code page */
  size_t meta_bytes;       /* device tables */
} lkv_size_info;

typedef struct {
  int32_t layer;             /* core layer */
  int32_t loop;              /* r, 0-based */
  int32_t n_seqs;            /* rows of q / out: 1..max_seqs */
  const int32_t* seq_ids;    /* host array [n_seqs] */
  int32_t q_len;             /* 1 for DECODE and DRAFT, k (<= max_block) for VERIFY */
  int32_t mode;              /* LKV_MODE_* */
  int32_t window;            /* RIPE window for this call; -1 = the cache's window */
  int32_t split_k;           /* splits of each row's pages; 0 = chosen by the library */
  float v_thresh_offset;     /* quant: far token hot iff s >= m0 - offset (m0 = max sink score) */
  const void* q;             /* device [n_seqs][q_len][n_heads_q][head_dim], kv dtype */
  void* out;                 /* device [n_seqs][q_len][n_heads_q][head_dim], kv dtype */
  float* lse;                /* device [n_seqs][q_len][n_heads_q] natural log, or NULL */
  void* workspace;           /* device scratch for split partials, lkv_workspace_bytes() */
  size_t workspace_bytes;
  /* DRAFT only: the draft block's own keys/values at this (layer, loop), for
     positions len..len+draft_len-1 of each sequence; the query is the last of
     them.  Device [n_seqs][draft_len][n_heads_kv][head_dim], kv dtype. */
  const void* draft_k;
  const void* draft_v;
  int32_t draft_len;         /* 1..max_block */
  /* Debug traces (NULL = off).  index_trace: device int32 [n_seqs][q_len][trace_len][2]
     holding (plane read, physical token slot = phys_page * 16 + slot) for every key
     position of query head 0, or (-1, -1) where the row does not read position j.
     mask_trace (quant): device uint32 [n_seqs][n_heads_q][ceil(n_far / 32)] hot bits. */
  int32_t* index_trace;
  int32_t trace_len;
  uint32_t* mask_trace;
  /* Optional hipEvent_t pair for timing the main attention kernel (not the merge):
     the launch itself stamps ev_begin with the kernel's start and ev_end with its
     end (hipExtLaunchKernel), so no marker packets are added to `stream`.  With
     more than 64 sequences the call launches one kernel per 64; ev_begin then marks
     the first one's start and ev_end the last one's end.  Either may be NULL. */
  void* ev_begin;
  void* ev_end;
  /* Quantised cells: hot-test rule (LKV_VRULE_*) and, for RUNNING, tau (the page uses 14). */
  int32_t v_rule;
  float v_tau;
  /* Launch shape; 0 = the library's default, measured best on MI355X at the workloads'
     shapes.  Wavefronts per workgroup of the attention kernel: multi-head decode and
     draft 2, 4 or 8 (default 8, or 4 for grouped-query heads), grouped-query decode tile
     1, 2 or 4 (default 4), verify 1, 2 or 4 (default 2), quantised cells 2 or 4 (default
     4).  Any other value is EINVAL.  The results do not depend on it. */
  int32_t waves;
  int32_t kernel;            /* LKV_KERNEL_* */
} lkv_attend_args;

typedef struct {
  int64_t logical_bytes;     /* K/V bytes the policy must hold: Eq. (3)/(10) core-layer terms */
  int64_t pages_in_use;      /* plain pages handed out */
  int64_t pages_total;
  int64_t code4_in_use, code4_total;
  int64_t code2_in_use, code2_total;
} lkv_mem_info;

typedef struct lkv_cache lkv_cache;

/* Page and table sizes for a configuration.  Pure host computation. */
lkv_status lkv_sizes(const lkv_config* cfg, lkv_size_info* out);

/* Create a cache over caller-owned arenas (host bookkeeping only; no device
   work).  Errors: EINVAL (config), ENOMEM (meta arena smaller than required). */
lkv_status lkv_create(const lkv_config* cfg, const lkv_arenas* arenas, int device, lkv_cache** out);
lkv_status lkv_destroy(lkv_cache* c);

/* Sequence slots.  A new sequence has length 0. */
lkv_status lkv_add_seq(lkv_cache* c, int32_t* seq_out);
lkv_status lkv_free_seq(lkv_cache* c, int32_t seq);

/* Allocate the pages that positions [pos0, pos0 + n_tok) of plane `plane` need,
   without writing them (host bookkeeping; lkv_append_plane = reserve + copy).
   Extends the sequence length to pos0 + n_tok.  Positions must not leave a gap
   after the plane's last position (ESTATE); RIPE non-deepest planes accept only
   positions >= committed - W that fit the window ring (EWINDOW).  Quantised caches
   hold the sink and the tail here: after the sink the far history may be skipped
   (supplied as code pages), and positions that already left the tail (encoded by
   lkv_window_exit) cannot be written again (ESTATE).  ENOMEM if the pool is empty. */
lkv_status lkv_reserve(lkv_cache* c, int32_t seq, int32_t layer, int32_t plane, int32_t pos0,
                       int32_t n_tok);

/* Write positions [pos0, pos0 + n_tok) of (seq, layer, plane): the keys and values
   that loop `plane` of core layer `layer` computed for those positions (RIPE page,
   Sec. 2: loop r of a core layer writes plane r; Algorithm 1, step 7: the emitted
   tokens' planes are appended to the cache, and step 5: the block's plane r exists by
   the time loop r attends).  k and v are device [n_tok][n_heads_kv][head_dim] in kv
   dtype, caller-owned, read on `stream`; the library copies them into its pages, so
   the caller may reuse them once the stream passes the call.  Quantised caches take
   the exact sink and tail positions here (LoopKV page, Sec. 3.2: sink and window stay
   exact bf16).  Errors as lkv_reserve, plus EDEVICE. */
lkv_status lkv_append_plane(lkv_cache* c, int32_t seq, int32_t layer, int32_t plane, int32_t pos0,
                            int32_t n_tok, const void* k, const void* v, void* stream);

/* The window slide of the RIPE page (Sec. 4 and Algorithm 1, step 7: drop planes
   1..R-1 of positions older than W): positions < new_len are committed, and the
   non-deepest planes of positions older than new_len - W are dropped (their
   window-ring pages return to the pool).  Commit is monotone: committed <= new_len
   <= length, else EINVAL (a window moved back would re-open positions whose ring
   pages are gone).  Quantised caches: host bookkeeping only; the tail's exit is
   lkv_window_exit. */
lkv_status lkv_commit(lkv_cache* c, int32_t seq, int32_t new_len);

/* Roll the sequence back to new_len positions: the rejected tail of a verified block
   (RIPE page, Algorithm 1, step 6: tokens past the accepted prefix and the verifier's
   token are not emitted, so step 7 appends nothing for them).  Pages holding only
   positions >= new_len return to the pool.  committed <= new_len <= length, else
   EINVAL. */
lkv_status lkv_truncate(lkv_cache* c, int32_t seq, int32_t new_len);

/* Quantised caches: the kind of every (layer, loop) cell, host int8
   [n_layers][n_loops] of LKV_CELL_INT4 / INT2 / SHARED.  The deepest loop may not
   be SHARED (EINVAL).  Must be set before any lkv_append_coded. */
lkv_status lkv_set_plan(lkv_cache* c, const int8_t* kinds);

/* Quantised caches: write far-history code pages [page0, page0 + n_pages) of
   (seq, layer, loop), already encoded by the caller ("LoopKV: Loop-Aware KV Cache
   Compression for Serving Looped Transformers", Sec. 3.1: KIVI-style codes with one
   fp16 scale and zero per group of 32, keys per channel and values per token;
   Sec. 3.3: INT4 value codes stored as a hi and a lo bit plane; Sec. 3.4: a page holds
   32 tokens of one (loop, layer) cell).  Far page p holds positions sink + 32p ..
   sink + 32p + 31.  The library packs the codes into its page layout.  The cell's
   encoded far history then extends to the end of page page0 + n_pages - 1.
   Inputs are device arrays in a plain logical layout (the library packs them):
     k_codes [n_pages*32][n_heads_kv][head_dim] uint8, values 0..2^bits-1;
     k_meta  [n_pages][n_heads_kv][head_dim][2] fp16 (scale, zero) per channel
             over the page's 32 tokens;
     v_codes [n_pages*32][n_heads_kv][head_dim] uint8;
     v_meta  [n_pages*32][n_heads_kv][head_dim/32][2] fp16 (scale, zero) per token
             and 32-channel group.
   bits = 4 for INT4 cells, 2 for INT2; SHARED cells store nothing (EINVAL). */
lkv_status lkv_append_coded(lkv_cache* c, int32_t seq, int32_t layer, int32_t loop, int32_t page0,
                            int32_t n_pages, const void* k_codes, const void* k_meta,
                            const void* v_codes, const void* v_meta, void* stream);

/* Quantised caches: the window-exit codec.  Encode far-history code pages
   [page0, page0 + n_pages) of (seq, layer, loop) from exact keys and values
   ("LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers",
   Sec. 3.1: KIVI-style codes, keys per channel over the page's tokens and values
   per token over 32 channels, each group with an fp16 scale and zero; Sec. 3.3:
   INT4 value codes stored as hi and lo bit planes).  Per group: scale =
   (max - min) / (2^bits - 1) in fp32, zero = min, both rounded to fp16 (nearest
   even); code = rint((x - zero16) / scale16) clamped to [0, 2^bits - 1], 0 when
   scale16 = 0.  bits follow the cell's plan (INT4 or INT2).
   k, v: device bf16 [(n_pages - 1) * 32 + n_valid_last][n_heads_kv][head_dim],
   caller-owned, holding positions sink + 32 page0 onwards; n_valid_last
   (1..32) = valid tokens of the last page (the rest get code 0 and zero
   metadata).  Errors as lkv_append_coded, plus EINVAL for n_valid_last. */
lkv_status lkv_encode_pages(lkv_cache* c, int32_t seq, int32_t layer, int32_t loop, int32_t page0,
                            int32_t n_pages, int32_t n_valid_last, const void* k, const void* v,
                            void* stream);

/* Quantised caches: the window exit ("LoopKV: Loop-Aware KV Cache Compression for
   Serving Looped Transformers", Sec. 3.4 and Sec. 4: when a page leaves the exact
   window, a KIVI codec quantises it into its cell's pool and the bf16 block is
   released; the quantisation runs before the step that reads it).  For sequence seq
   of length L, the far history is [sink, L - tail): every far position that left the
   tail since the last exit is encoded, in every INT4 and INT2 cell, from the cell's
   own exact plane (appended with lkv_append_plane) into its code pages with the codec
   of lkv_encode_pages; a partially filled last code page is encoded again from all its
   valid tokens, so the codes always equal the codec applied to the page's exact
   values.  Exact pages that no cell reads any more return to the pool: pages wholly
   past the sink whose positions lie in complete code pages (or, for a shared cell,
   that all left the tail).  Call it after appending a step's tokens and before the
   step's attend calls; positions that left the tail can no longer be appended or
   truncated.  Device work on `stream`.  Errors: ESTATE (not a quantised cache, no
   plan, an exact page missing), ENOMEM (code pools exhausted; nothing changed),
   EDEVICE. */
lkv_status lkv_window_exit(lkv_cache* c, int32_t seq, void* stream);

/* Quantised caches: read code pages back into the logical layout lkv_append_coded
   takes (the inverse of its packing), into caller-owned device buffers of the
   same shapes: the page contents of LoopKV page Sec. 3.1 and 3.3-3.4 (codes, fp16
   scale and zero, hi and lo planes merged back into one code), for byte checks of
   the codec.  Errors: EINVAL (arguments, shared cell), ESTATE (page not
   resident), EDEVICE. */
lkv_status lkv_read_coded(lkv_cache* c, int32_t seq, int32_t layer, int32_t loop, int32_t page0,
                          int32_t n_pages, void* k_codes, void* k_meta, void* v_codes, void* v_meta,
                          void* stream);

/* Workspace an attend call needs (0 when it runs unsplit).  For a quantised cache the
   library's split choice depends only on the batch (sequences, heads, far lengths), so
   the size covers the call's (layer, loop) whatever its cell kind and V-precision rule,
   and one buffer serves every cell call of that batch. */
lkv_status lkv_workspace_bytes(const lkv_cache* c, const lkv_attend_args* a, size_t* bytes);

/* Attention of n_seqs rows at (layer, loop), on `stream`: for query position t,
   out = softmax(q k_j / sqrt(d)) v over keys j <= t, each key read from the plane
   the policy names (RIPE page, Sec. 2 policy pi and Eq. (9); positions of the
   query's own block read plane r, proof of Prop. 1), lse = natural log of the
   softmax denominator.
   DECODE (q_len = 1) and VERIFY (q_len = k, causal inside [t0, L); RIPE page,
   Algorithm 1, step 5: one R-loop pass over the block) read the cache; with
   W >= k - 1 a verify equals k sequential decodes (Prop. 1).  DRAFT (Algorithm 1,
   steps 2-4) reads cached positions < len through the policy with the given
   window (0 = the deepest plane, as the page's drafts read) and the block's
   positions from draft_k / draft_v.  Quantised caches serve DECODE over their
   cells (LoopKV page, Sec. 3.1-3.4 and App. E Algorithm 1: exact sink and tail,
   INT4 / INT2 / shared far history, V lo plane read only for hot tokens).
   Splits of a row's pages are merged exactly by log-sum-exp (LoopKV page,
   Sec. 3.4).  Workspace, outputs and traces are caller-owned device memory.
   Errors: EINVAL (arguments), ESTATE (a needed page is missing), ENOMEM
   (workspace too small), EUNSUPPORTED, EDEVICE. */
lkv_status lkv_attend(lkv_cache* c, const lkv_attend_args* a, void* stream);

/* lkv_attend for callers that cannot allocate device memory or pass a workspace: code
   under HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same
   arguments, checks, kernels and results as lkv_attend, except that workspace must be
   NULL and workspace_bytes 0: the split partials go to a fixed device array of
   LKV_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the
   process ends.  A call whose partials would not fit is refused (EINVAL) before any
   device work.  Nothing is allocated (no hipMalloc, hipFree or allocating library
   routine).  Every call on one GPU uses that GPU's one array, so calls that overlap on
   the same GPU (other streams, other threads, other handles) race and must be
   serialised by the caller.  The handle's device must be current.  Errors as
   lkv_attend, plus EDEVICE if the array's address cannot be resolved. */
#define LKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
lkv_status lkv_attend_noalloc(lkv_cache* c, const lkv_attend_args* a, void* stream);

lkv_status lkv_mem_stats(const lkv_cache* c, lkv_mem_info* out);

/* Host index function: the plane, physical page and slot that the row at
   position t of a block starting at t0 reads for key j (window -1 = cache
   default), by RIPE page Sec. 2 policy pi and Eq. (9) with the block rule of the
   proof of Prop. 1.  -1 for a page that is not resident. */
lkv_status lkv_debug_resolve(const lkv_cache* c, int32_t seq, int32_t layer, int32_t loop, int32_t t,
                             int32_t t0, int32_t j, int32_t window, int32_t* plane,
                             int32_t* phys_page, int32_t* slot);

/* Length and committed length of a sequence. */
lkv_status lkv_seq_info(const lkv_cache* c, int32_t seq, int32_t* len, int32_t* committed);

/* Measurement aid, not a step of the attention path: one streaming read of
   `bytes` bytes of device memory at `buf` with the load form the page streams
   use (16-byte nontemporal loads, each wave instruction covering a whole 1 KB
   run), on `stream`.  Its rate is the achievable HBM read bandwidth that the
   attention kernels are compared with.  `bytes` must be a positive multiple of
   LKV_PROBE_CHUNK (below 2^31 chunks); `sink` is one caller-owned device word
   that the kernel may overwrite.  ev_begin / ev_end (hipEvent_t, may be NULL)
   are stamped with the start and end of the kernel's own dispatch, as the
   attend call's timing events are.  No handle is involved.  Errors: EINVAL
   (NULL pointer or bad size), EDEVICE (launch failed). */
#define LKV_PROBE_CHUNK 16384
lkv_status lkv_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* ev_begin, void* ev_end,
                          void* stream);

const char* lkv_last_error(const lkv_cache* c);
const char* lkv_status_str(lkv_status s);

#ifdef __cplusplus
}
#endif

#endif /* LOOPATTN_H */
