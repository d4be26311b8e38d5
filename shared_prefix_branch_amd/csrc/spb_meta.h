// spb_meta.h -- the device metadata of one packed pass (internal to libspb).
//
// One contiguous blob, built by the host planner and copied to device memory
// once per pass: a header, then arrays each starting on a 256-byte boundary.
// Every kernel reads only this blob plus the caller's tensors.
//
// Including translation units define SPB_HD first: `__host__ __device__` in
// HIP sources, empty in host-only C++.
#pragma once
#include <stdint.h>

#ifndef SPB_HD
#error "define SPB_HD before including spb_meta.h"
#endif

namespace spb {

constexpr int32_t kMetaMagic = 0x53504231;  // "SPB1"
constexpr int32_t kMetaVersion = 3;
constexpr int kTileRows = 128;  // rows per attention tile (one to two work groups)
constexpr int kChunk = 64;      // keys per content chunk, chunks start at the content start
constexpr int kBranchChunk = 32;  // keys per branch chunk, chunks start at the branch start
constexpr int kMaxTileChunks = 320;  // key chunks one attention tile may visit
constexpr int kMaxDepth = 4;    // option-trie depth (options of at most 5 tokens)
constexpr int kVocabTile = 256; // vocabulary rows per lm-head slice (LSE partial)

// One per pass row.  Visibility of key row y from query row x:
//   content key: y in [x.seg, x.seg + x.cvis)
//   stem key (a shared template token, of stem s with DFS interval
//     [pre_s, post_s)): visible iff pre_s <= x.spre < post_s, and, when x is
//     a row of s itself (x.stem and y in s), iff y <= x (causal)
//   branch key:  x.br >= 0, !x.stem and y in [x.br, x.br + E) with e' = y - x.br:
//     e' <  x.L : visible iff e' <= x.e  (template rows causal; nodes see all)
//     e' >= x.L : visible iff e' is one of the node's ancestors anc[0..depth)
struct SpbRow {
  int32_t cvis;   // content keys visible (content row t: t+1; branch and stem rows: C)
  int32_t seg;    // pass row of the segment's first content token
  int32_t br;     // pass row of the branch's own template token 0 (stem rows: of the
                  // stem's first token); -1 for content rows
  int32_t e;      // extended index in the branch or stem (template j or L + node index); content: t
  int32_t L;      // own template length of the branch, or the stem's length (0 for content rows)
  int32_t depth;  // option-trie depth (0 for content, template and stem rows)
  int32_t anc01;  // extended indices of ancestors at depth 1 and 2 (low / high 16 bits)
  int32_t anc23;  // depth 3 and 4; anc[depth-1] is the node itself
  int32_t spre;   // pre number of the deepest stem on the row's path (its own stem for a
                  // stem row); -1: none
  int32_t stem;   // 1 for a stem row
  int32_t pad0, pad1;
};

// One attention work item: at most kTileRows consecutive rows of one segment
// (or of a run of empty-content floor branches).
struct SpbTile {
  int32_t row0, nrows;
  int32_t seg;    // content start (pass row) shared by the tile's rows
  int32_t ncc;    // content chunks to visit: ceil(max cvis / kChunk)
  int32_t b_lo, b_hi;  // branch-table range intersecting the tile
  int32_t cost;        // key chunks the tile visits (content + branch)
  int32_t pad;
};

// One work item of the bf16 attention kernel at a row granularity of 32 << g
// (g = 0, 1, 2): rows [row0, row0 + nrows) of one tile, the content chunks
// its rows see (chunk c holds content keys [64c, 64c + 64)), and the branch
// chunks of the branches meeting its rows, entries [boff, boff + bn) of the
// pass's branch-chunk list.  Items of one granularity are ordered longest
// first (cost = ncc + bn).
struct SpbItem {
  int32_t row0, nrows;
  int32_t seg;    // content start (pass row)
  int32_t ncc;    // content chunks: ceil(max cvis over the item's rows / kChunk)
  int32_t boff, bn;
  int32_t cost, pad;
};

// A branch chunk: keys [key0, key0 + kBranchChunk) of branch `b`, chunk c of
// it (key0 = start + c * kBranchChunk); info = b << 10 | c.  A stem chunk:
// keys [key0, key0 + kBranchChunk) of stem s, info = kStemChunk | s << 10 | c,
// pre / post its DFS interval, nvis its keys (up to kBranchChunk; all of them
// are seen by a row below the stem).
constexpr int32_t kStemChunk = 1 << 30;
struct SpbChunk {
  int32_t key0, info;
  int32_t pre;
  int32_t post_nvis;  // post | nvis << 24
};

struct SpbBranch {
  int32_t start;   // pass row of template token 0
  int32_t L, E;    // template length; template + trie nodes
  int32_t n_opt;   // options of the question
  int32_t opt0;    // first option slot of the pass
  int32_t scored0; // scored-row index of the template's last row (nodes follow)
  int32_t n_scored;
  int32_t question;
};

struct SpbMetaHeader {
  int32_t magic, version;
  int32_t pass, n_tokens;
  int32_t n_tiles, n_branches, n_options, n_scored;
  int32_t n_targets, n_steps, pad0, pad1;
  int64_t off_rows, off_tiles, off_branches, off_scored;
  int64_t off_tgt_off, off_tgt_tok, off_opt_step_off, off_step_slot;
  int64_t off_step_row, total_bytes, pad2, pad3;
  int64_t off_items[3], off_bchunks;  // work items at 32, 64, 128 rows; their branch chunks
  int32_t n_items[3], n_bchunks;
};

SPB_HD inline int anc_of(const SpbRow &r, int i) {
  int32_t w = i < 2 ? r.anc01 : r.anc23;
  return (i & 1) ? (int)((uint32_t)w >> 16) : (int)(w & 0xFFFF);
}

// Is branch key with extended index ep visible from row r (r in that branch)?
SPB_HD inline bool branch_visible(const SpbRow &r, int ep) {
  if (ep < r.L) return ep <= r.e;
  bool v = false;
  for (int i = 0; i < kMaxDepth; ++i) v = v || (i < r.depth && anc_of(r, i) == ep);
  return v;
}

}  // namespace spb
