// Kernel parameter blocks shared by the host library and the HIP kernels.
// Passed by value as kernel arguments (well under the 4 KB limit).
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace lkv {

constexpr int kPage = 16;       // tokens per plain page
constexpr int kQuad = 4;        // tokens interleaved per channel in a V block
constexpr int kCodePage = 32;   // tokens per code page
constexpr int kMaxRows = 64;    // sequences per launch
constexpr int kMaxBlock = 16;   // verify rows per sequence (one MFMA tile)

enum : int32_t { kFull = 0, kRipe = 1 };
enum : int32_t { kDecode = 0, kVerify = 1, kDraft = 2 };

// Plain page layout (one page = one (seq, layer, plane), all KV heads, 16 tokens):
//   K block: [head][token 0..15][channel 0..D-1]
//   V block: [head][quad g 0..3][channel 0..D-1][i 0..3], entry i of quad g = token 4 i + g
// so each (page, head) K slice and V slice is one contiguous run of 16*D elements.
// V interleaves four tokens per channel: a lane reads four tokens of two (bf16) or one
// (fp32) channel in one 16-byte load, and the verify tile gets its V^T operand
// directly.  A quad holds every fourth token so that the decode kernel, whose DPP
// row g handles the tokens 4 i + g, reads K four whole token rows per load
// instruction (whole 128-byte lines) and V whole 256-byte runs per instruction.

// Attention over plain pages (DECODE, VERIFY, DRAFT).
struct PlainParams {
  const uint8_t* pool;        // plain page arena
  uint64_t page_bytes;
  const int32_t* tab_own;     // table of the loop's own plane: [seq slot][ring_own]
  const int32_t* tab_deep;    // table of the deepest plane:    [seq slot][ring_deep]
  int32_t ring_own;
  int32_t ring_deep;
  const void* q;              // [n_rows][q_len][hq][D]
  void* out;                  // [n_rows][q_len][hq][D]
  float* lse;                 // [n_rows][q_len][hq] or null
  float* ws;                  // split partials [n_rows][q_len][hq][n_splits][D + 1]
  const void* draft_k;        // DRAFT: [n_rows][draft_len][hkv][D]
  const void* draft_v;
  int32_t* trace;             // [n_rows][q_len][trace_len][2] or null
  int32_t trace_len;
  int32_t draft_len;
  int32_t n_rows, q_len, hq, hkv;
  int32_t window;             // effective RIPE window
  int32_t ripe;               // 1: RIPE with loop < deepest; 0: every position reads tab_own
  int32_t loop;
  int32_t deepest;
  int32_t n_splits;
  float scale_log2;           // log2(e) / sqrt(D)
  int32_t slot[kMaxRows];     // sequence slot (row of the tables)
  int32_t len[kMaxRows];      // cached positions of the sequence
};

// Quantised LoopKV-style cells (DECODE).
struct CellParams {
  const uint8_t* pool;        // plain (bf16) pages: sink and tail of the cell's own loop
  uint64_t page_bytes;
  const int32_t* tab_near;    // [seq slot][ring_near]
  int32_t ring_near;
  const uint8_t* codes;       // code page arena of the cell's source (own, or the final loop's)
  uint64_t code_page_bytes;
  const int32_t* tab_code;    // [seq slot][code_ring]
  int32_t code_ring;
  int32_t bits;               // 4 or 2
  int32_t masked;             // 1: V lo plane read only for hot tokens (INT4 / shared cells)
  float thr_offset;           // rule 0: hot iff s >= m0 - thr_offset (natural-log units)
  int32_t rule;               // 0: fixed offset from m0; 1: running maximum (LoopKV page, App. E Alg. 1)
  float v_tau;                // rule 1: hot iff s log2(e) >= max(m, m0) log2(e) - v_tau
  const void* q;
  void* out;
  float* lse;
  float* ws;                  // partials [n_rows][hq][n_splits + 1][D + 1]
  uint32_t* mask_trace;       // [n_rows][hq][mask_words] or null
  int32_t mask_words;
  int32_t n_rows, hq, hkv;
  int32_t sink, tail;
  int32_t n_splits;           // far splits; block x == n_splits is the near (sink + tail) block
  float scale_log2;
  float scale;                // 1 / sqrt(D)
  int32_t slot[kMaxRows];
  int32_t len[kMaxRows];
};

// Merge of split partials.
struct MergeParams {
  const float* ws;            // [rows][n_parts][D + 1], entry D = base-2 lse (-inf if empty)
  void* out;                  // [rows][D]
  float* lse;                 // [rows] or null
  int32_t n_rows;
  int32_t n_parts;
};

// Pack logical code arrays into up to 64 code pages (lkv_append_coded).
struct PackParams {
  uint8_t* arena;             // code page arena of the cell's kind
  uint64_t page_bytes;
  const uint8_t* k_codes;     // [n_pages * 32][hkv][D]
  const uint16_t* k_meta;     // [n_pages][hkv][D][2]
  const uint8_t* v_codes;     // [n_pages * 32][hkv][D]
  const uint16_t* v_meta;     // [n_pages * 32][hkv][D / 32][2]
  int32_t hkv, bits;
  int32_t n_pages;
  int32_t phys[64];           // physical page of batch page i
};

// Encode exact bf16 keys and values of up to 64 far pages into code pages (the
// window-exit codec).  The values come either from caller arrays (k, v) or, when
// tab_plain is set, from the cell's own plain pages (the tail the positions leave).
struct EncodeParams {
  uint8_t* arena;
  uint64_t page_bytes;
  const uint16_t* k;          // bf16 [n_pages * 32][hkv][D]
  const uint16_t* v;
  const uint8_t* pool;        // plain page arena, when reading from pages
  uint64_t plain_page_bytes;
  const int32_t* tab_plain;   // the sequence's row of the plain table, or null
  int32_t pos0;               // position of token 0 of batch page 0 (sink + 32 page0)
  int32_t hkv, bits;
  int32_t n_pages;
  int32_t n_valid_last;       // valid tokens of the last page (1..32)
  int32_t phys[64];
};

// Write up to kTableChunk int32 block-table entries (values passed by value, so no
// host-to-device copy of pageable memory is needed and the write is a plain kernel).
constexpr int kTableChunk = 960;
struct TableWriteParams {
  int32_t* dst;
  int32_t n;
  int32_t vals[kTableChunk];
};

// Append rows into plain pages.
struct CopyParams {
  uint8_t* pool;
  uint64_t page_bytes;
  const void* k;              // [n_tok][hkv][D]
  const void* v;
  int32_t pos0, n_tok, hkv;
  int32_t page0;              // logical page of pos0
  int32_t n_pages;
  int32_t phys[64];           // physical page of logical page page0 + i
};

}  // namespace lkv
