// Host planner for the attention kernels: from the block tables of a batch
// of sequences to segments (runs of blocks shared by the same set of
// sequences), chunks and work items, plus the per-branch list of partial
// states the combine step merges. See attn_plan.h for the device-side records.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "pool.hpp"
#include "attn_plan.h"

namespace pkv {

struct SchedOptions {
  int32_t chunk_tokens = 0;        // 0 = automatic
  int32_t rows_per_item = 32;      // narrow items (16 on the VALU path)
  bool wide = true;                // chunks with more rows go to wide items
  int32_t wide_rows = 256;         // rows per wide item at most (also capped by the kernel shape)
  bool wide_fill = true;           // wide items full but the last (else an even split)
  int32_t target_workgroups = 256;  // shorten chunks while the grid has fewer than 3/4 of this
  // shortest automatic chunk, and chunk length per query row (keeps the
  // partial states ~3% of the K/V bytes); 0: by head size (1024 and 64 up to
  // D = 128, 768 and 32 above: a 256-dim step is twice the bytes, and a
  // wave's chain of dependent steps is what bounds a long narrow item)
  int32_t min_chunk_tokens = 0;
  int32_t max_chunk_tokens = 8192;
  int32_t tokens_per_row = 0;
  // 16-row blocks one narrow wave may own: 1, 2, or 0 for automatic (2 when
  // items of more than 16 rows hold at least a quarter of the narrow tokens)
  int32_t max_row_blocks_per_wave = 0;
  bool short_items = true;         // one wave per plane for short narrow items
  int32_t short_tokens = kShortTokens;  // longest narrow item (of <= 16 rows) that counts as short
  int32_t fold_tokens = 64;        // shared segments shorter than this are read per branch (0: never)
  bool finalize = true;            // the narrow launch may write final outputs (see Schedule::finalize)
  // Rows of one grouped item at most (0: no grouping): after folding, the
  // runs of sibling branches that share blocks are served by one item of
  // group_rows / G branches, which reads each of their blocks once and
  // masks it for the rows whose branch does not hold it. At most 16 (one
  // row block) and at most rows_per_item.
  int32_t group_rows = 16;
  // Tree launch (one workgroup per plane holding every row and reading each
  // chunk once): 0 never, 1 when it applies and pays (all rows fit one
  // workgroup, some segment has more rows than a narrow item, and the planes
  // alone fill the chip), 2 whenever it applies (for tests). Off by
  // default: on the MCTS batch the tree launch measures slower than the
  // wide and narrow launches together. tree_ok: the head size and dtype
  // have a tree kernel.
  int32_t tree = 0;
  bool tree_ok = false;
  int32_t tree_piece_tokens = 512;  // the widest segments are cut into pieces of this many tokens
};

struct Schedule {
  std::vector<WorkItem> items;     // narrow items (long, then short), then wide items
  int32_t n_narrow = 0;
  int32_t n_short = 0;             // short narrow items (the last n_short of the narrow ones)
  bool folded = false;             // short shared segments were folded into per-branch items
  bool grouped = false;            // some item serves a group of branches (binfo is filled)
  // long narrow items dealt by plane as the short ones of a folded plan are
  // (n_long_wgs counts the padded grid part); matrix-core launch only
  bool long_by_plane = false;
  int32_t n_long_wgs = 0;
  // Every branch has exactly one chunk read by narrow items and its other
  // chunks by wide items: the wide launch runs first, so each narrow row can
  // merge its branch's wide partials itself and write the output (no combine).
  bool finalize = false;
  // The tree launch serves the whole batch (titems / tchunks); no narrow or
  // wide items, no partial states, no combine.
  bool tree = false;
  std::vector<TreeItem> titems;
  std::vector<TreeChunk> tchunks;
  int32_t narrow_rw = 1;           // 16-row blocks per wave in the narrow launch
  std::vector<int32_t> order;      // workgroup order of the wide launch
  int32_t n_order_narrow = 0;      // workgroups of the narrow launch (no table)
  int32_t n_order_wide = 0;
  std::vector<int32_t> blk;
  // parallel to blk when grouped: holder bits of the block within its item
  // (bit h: the item's holder h reads it) | valid slots << 16; 0 on padding
  std::vector<int32_t> binfo;
  std::vector<int32_t> holders;
  std::vector<int32_t> comb_ptr;
  std::vector<int32_t> comb_rows;
  std::vector<uint64_t> anc;
  int32_t P = 0;         // partial rows per (layer, KV head) plane
  int32_t n_branch = 0;  // query rows' branches (sequences, or requests x nodes)
  int32_t n_layers = 0;
  int32_t n_segments = 0;
  int32_t n_chunks = 0;
  int64_t unique_tokens = 0;  // distinct (block, slot) token positions read per plane
  int64_t wide_tokens = 0;    // of those, the ones in chunks served by wide items

  // byte offsets inside the workspace
  size_t off_items = 0, off_blk = 0, off_holders = 0, off_comb_ptr = 0, off_comb_rows = 0,
         off_anc = 0, off_order = 0, off_titems = 0, off_tchunks = 0, off_binfo = 0,
         meta_bytes = 0, off_ml = 0, off_acc = 0, total_bytes = 0;

  void layout(int Hkv, int D);
  // Fills `order` for n_layers x Hkv planes (items must be final).
  void build_order(int32_t n_layers, int32_t Hkv);
  void pack_meta(uint8_t* dst) const;  // writes meta_bytes bytes
};

// Scratch arrays sized by the pool's block count, reused between calls.
struct PlannerScratch {
  std::vector<uint32_t> stamp;
  std::vector<int32_t> cnt, pos, valid, off, fill, seg;
  uint32_t epoch = 0;
  void ensure(int nb);
};

int build_decode_schedule(const Pool& pool, const pkv_seq* seqs, int32_t n, int32_t n_layers,
                          int32_t layer0, const SchedOptions& opt, PlannerScratch* scratch,
                          Schedule* out);

int build_verify_schedule(const Pool& pool, const pkv_seq* reqs, int32_t n_req,
                          const int32_t* parents, int32_t n_nodes, const SchedOptions& opt,
                          Schedule* out);

}  // namespace pkv
