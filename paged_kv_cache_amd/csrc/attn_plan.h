// Attention schedule shared by the host planner (schedule.cpp) and the
// device kernels (kernels.hip). Plain data, int32 indices.
//
// A *segment* is a maximal run of blocks that the same set of sequences
// (its holders) reference at the same logical positions; forks share
// prefixes, so the segments of a batch form a tree. A segment is cut into
// *chunks* of whole blocks, and a chunk's rows (holder x query head of one
// KV-head group) are cut into *work items*: narrow items of up to 32 rows
// or wide items of up to 128 rows. Every work item runs once per (layer, KV
// head); an order table maps workgroups to (item, layer, head) so that the
// wide items of one chunk land on the same XCD, next to each other in
// dispatch order, and share its L2.
#pragma once

#include <cstdint>

namespace pkv {

// Most blocks one chunk may span: the matrix-core kernels copy a chunk's
// block ids to LDS.
constexpr int32_t kMaxChunkBlocks = 512;

// A narrow item of at most 16 rows and this many tokens is short: one wave
// does all of it (four items' planes per workgroup) instead of four waves
// splitting its steps and merging. (A four-wave item pays its start-up
// chain of dependent loads and the merge for every few steps it loads.)
constexpr int32_t kShortTokens = 256;
// Largest schedule (all its arrays, 16-byte aligned) that a launch carries in
// its own arguments, and the same for the combine's lists. Kernel arguments
// are written by the runtime as part of the dispatch, so such a call needs no
// separate host-to-device copy before its first launch. (By-value arguments
// of 3 to 16 KiB reached the device intact on this runtime; at 12 KiB the
// MCTS plan, 8 KB, travels this way: 0.328-0.330 -> 0.324 ms per call, the
// beam step unchanged.)
constexpr int32_t kInlineMetaBytes = 12288;
constexpr int32_t kInlineListBytes = 1024;

struct WorkItem {
  int32_t blk_off;    // index in blk[] of the chunk's first block
  int32_t n_tok;      // valid tokens in the chunk (> 0)
  int32_t t0;         // logical position of the chunk's first token
  int32_t hold_off;   // index in holders[] of the chunk's first holder
  int32_t r0;         // first chunk row handled (chunk row = holder * G + g)
  int32_t n_rows;     // rows handled by this item (1 .. 64)
  int32_t part_row;   // partial-state row of this item's first row, per plane
  int32_t mask_from;  // first logical position under the draft-tree mask (INT32_MAX: none)
  int32_t reread;     // 1: another item (or another wave) reads the same chunk, so K/V
                      // go through the caches; 0: streaming loads
  int32_t grouped;    // 0, or the holder bits of all the item's holders: the chunk is a
                      // group of branches' blocks, each masked by its binfo word
  int32_t pad[2];
};
static_assert(sizeof(WorkItem) == 48, "WorkItem layout");

// Tree items (decode of a batch whose rows all fit one workgroup): one
// workgroup per (tree item, layer, KV head) holds up to kTreeRows query rows
// (row r = holder r / G, q-head offset r % G) and reads every chunk any of
// them holds, each once, applying it to the rows that hold it; it writes
// the final output rows (no partial states, no combine).
constexpr int32_t kTreeRows = 256;
constexpr int32_t kMaxTreeBlocks = 2048;  // block ids of an item, staged in LDS
constexpr int32_t kMaxTreeChunks = 256;   // chunk records of an item, staged in LDS

struct TreeItem {
  int32_t hold_off;   // index in holders[] of the item's first holder
  int32_t n_rows;     // query rows (1 .. kTreeRows)
  int32_t chunk_off;  // index of the item's first TreeChunk
  int32_t n_chunks;
  int32_t blk_off;    // index in blk[] of the item's first block id
  int32_t n_blk;      // block ids of all its chunks (<= kMaxTreeBlocks)
  int32_t n_steps;    // 32-token steps over all its chunks
  int32_t pad;
};
static_assert(sizeof(TreeItem) == 32, "TreeItem layout");

struct TreeChunk {
  int32_t blk_off;    // first block id, relative to the item's blk_off; padded to whole steps
  int32_t n_tok;      // valid tokens (> 0)
  int32_t t0;         // logical position of the first token
  int32_t n_steps;    // ceil(n_tok / 32)
  uint64_t rows[4];   // bit r % 64 of rows[r / 64]: item row r reads this chunk
};
static_assert(sizeof(TreeChunk) == 48, "TreeChunk layout");

// Device-side pointers to a decode / verify schedule and its partials.
// Partial states are stored per plane (layer, KV head): P rows each.
struct AttnCore {
  const void* k_arena;      // [L][NB][Hkv][BS][D]
  const void* v_arena;      // [L][NB][Hkv][D][BS]
  const void* q;            // [n_layers][n_branch][Hq][D]
  float* part_ml;           // [n_layers * Hkv][P][2]: running max (log2 units), sum
  float* part_acc;          // [n_layers * Hkv][P][D]
  // The schedule's arrays sit at byte offsets from one base: the PlanBytes
  // passed with the launch when meta_inline (a small schedule then travels
  // with the launch itself and no upload precedes it), else meta_dev in the
  // workspace.
  //   items    WorkItem[n_items]
  //   blk      block ids, per chunk padded to a whole 32-token step
  //   holders  branch index of each holder
  //   anc      uint64 [n_branch] ancestor-or-self bits (verify only)
  //   order    wide launch: per workgroup item * (n_layers * Hkv) + layer * Hkv + head, or -1
  //   comb_ptr [n_branch + 1], comb_rows: each branch's partial rows (q-head offset 0) in logical order
  //   titems   TreeItem[], tchunks TreeChunk[] (tree launch only)
  //   binfo    parallel to blk (grouped items only): holder bits | valid slots << 16
  const uint8_t* meta_dev;
  int32_t meta_inline;
  int32_t off_items, off_blk, off_holders, off_anc, off_order, off_comb_ptr, off_comb_rows;
  int32_t off_titems, off_tchunks, off_binfo;
  int32_t n_order;          // workgroups in the launch
  // Narrow launch (no order table): code = item * (n_layers * Hkv) + layer *
  // Hkv + head. Workgroups [0, n_long) take code = blockIdx; after them each
  // workgroup takes four codes of short items, one per wave.
  int32_t n_long;
  int32_t n_long_wgs;       // workgroups of the long items (padded when long_by_plane)
  int32_t long_by_plane;    // long items: a plane's items in consecutive rounds of one XCD
  int32_t n_codes;
  int32_t short_by_plane;   // short workgroups take four items of one plane (else four planes of one item)
  // With finalize, the narrow launch runs after the wide one and each of its
  // rows merges its branch's other partial states (comb_ptr / comb_rows, as
  // the combine reads them) and writes the output row instead of a partial.
  int32_t finalize;
  float* out;               // [n_layers][n_branch][Hq][D]
  int32_t n_items;
  int32_t n_layers;
  int32_t layer0;
  int32_t num_blocks;
  int32_t Hkv;
  int32_t G;
  int32_t Hq;
  int32_t n_branch;
  int32_t P;
  float scale_log2;         // softmax scale * log2(e)
  // The wide kernel takes scores unscaled and folds the scale into the
  // exponent: max(|scale| * log2(e), 1e-30) (a zero scale becomes a tiny
  // one, so that a masked -inf score still gives 0), with q's sign bits
  // flipped (q_flip = 0x80008000 on bf16 pairs) when the scale is negative.
  float abs_scale_log2;
  uint32_t q_flip;
};

// The inline schedule bytes: the kernels take them as a second argument
// beside AttnCore, so that copies of the small part never carry them.
struct PlanBytes {
  alignas(16) uint8_t b[kInlineMetaBytes];
};

struct AttnParams : AttnCore {
  PlanBytes meta;
};

struct CombineParams {
  const float* part_ml;
  const float* part_acc;
  // comb_ptr [n_branch + 1] and comb_rows (partial row of q-head group
  // offset 0, in logical order) at byte offsets from `lists` when
  // lists_inline, else from meta_dev
  const uint8_t* meta_dev;
  int32_t lists_inline;
  int32_t off_comb_ptr, off_comb_rows;
  float* out;                // [n_layers][n_branch][Hq][D]
  int32_t n_layers;
  int32_t n_branch;
  int32_t Hkv;
  int32_t G;
  int32_t Hq;
  int32_t P;
  alignas(16) uint8_t lists[kInlineListBytes];
};

}  // namespace pkv
