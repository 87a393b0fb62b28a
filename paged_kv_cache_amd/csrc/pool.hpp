// Host side of the paged KV cache: the block pool with reference counts,
// per-sequence block tables, fork, free and the append planner with
// copy-on-write. Plain C++17, no HIP: every call here is integer work on the
// host and is all-or-nothing.
//
// Mechanism (Dendrite author's replies): KV memory is paged in fixed-size
// blocks; a fork is a shallow copy of the block table through copy-on-write;
// a block being written must never be aliased, so an append into a shared,
// partly filled tail block first copies it.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "pkv.h"

namespace pkv {

// Sets `msg` as this thread's last error and returns `code`.
int fail(int code, const std::string& msg);
void clear_error();
const char* last_error();

// Free set over allocation ranks: a bitset with summary levels, so taking
// the lowest free rank and returning one are O(levels) word operations.
class FreeSet {
 public:
  void init(int n);  // all ranks free
  int count() const { return count_; }
  int pop_lowest();  // -1 if empty
  void insert(int rank);
  void erase(int rank);  // rank must be free
  bool contains(int rank) const;

 private:
  std::vector<std::vector<uint64_t>> lv_;  // lv_[0] leaf bits, lv_[k+1] = nonzero words of lv_[k]
  int n_ = 0;
  int count_ = 0;
};

// Block tables are persistent and shared: a sequence points at a table
// list (refcounted), the list at table chunks (refcounted, up to kChunk
// block ids each). A fork copies the list pointer and bumps one count; a
// list or chunk is copied only when a sequence that shares it is about to
// change it. A block's count (ref_) counts the chunks and prompt-cache
// entries that hold it; what a caller sees (pkv_block_refcount) is the
// number of sequences and entries that hold it, as before. A block is
// written in place only if neither its sequence's list, nor its chunk, nor
// the block itself is shared.
constexpr int32_t kChunk = 64;

struct TChunk {
  int32_t ref = 0;
  int32_t n = 0;
  int32_t ids[kChunk];
};

struct TList {
  int32_t ref = 0;
  std::vector<int32_t> chunks;
};

struct Seq {
  uint32_t gen = 1;
  bool live = false;
  int32_t len = 0;
  int32_t list = -1;  // -1: no blocks
  // the table flattened, built on demand and dropped when the table changes
  mutable std::vector<int32_t> flat;
  mutable bool flat_ok = true;
};

// A prompt-cache entry: one full block, keyed by its token ids and the
// entry of the block before it (so a chain from the root spells a prefix).
struct CacheEntry {
  int32_t parent = -1;  // entry id, -1 at the root
  int32_t block = -1;
  int32_t depth = 0;    // 1 for a prompt's first block
  int32_t n_child = 0;  // live entries whose parent this is
  uint64_t stamp = 0;   // the last insert or match that walked it
  uint64_t hash = 0;
  bool live = false;
};

class Pool {
 public:
  explicit Pool(const pkv_pool_desc& d);

  const pkv_pool_desc& desc() const { return d_; }
  int block_size() const { return d_.block_size; }

  int block_alloc(int32_t* id);
  int block_release(int32_t id);

  int seq_create(pkv_seq* out);
  int seq_fork(pkv_seq parent, pkv_seq* child);
  int seq_free(pkv_seq s);
  // Keeps the first n tokens (0 <= n <= len): blocks that then hold none of
  // the sequence's tokens lose its reference; a kept partly filled block
  // keeps its count.
  int seq_truncate(pkv_seq s, int32_t n);
  // Truncates s to keep_len tokens, then plans an append of n_new tokens;
  // if the append is refused, the truncation is undone (all or nothing).
  int truncate_append(pkv_seq s, int32_t keep_len, int32_t n_new, std::vector<int64_t>* slots,
                      std::vector<pkv_cow_op>* cows);
  // The same for n distinct sequences: all are truncated, then one batch
  // append plans seqs[i] += n_new[i] in order; if it is refused, every
  // truncation is undone.
  int truncate_append_batch(const pkv_seq* seqs, const int32_t* keep_lens, const int32_t* n_new,
                            int32_t n, std::vector<int64_t>* slots, std::vector<pkv_cow_op>* cows);

  // Prompt cache (Ferrite page, section 07: resume from the longest match;
  // parked conversations keep their blocks). Entries hold one reference on
  // their block. The next entry evicted is, among leaf entries whose block
  // only the cache holds, the one with the oldest stamp (deepest on a tie).
  // An allocation that finds no free block evicts one entry first.
  int prefix_insert(pkv_seq s, const int32_t* tokens, int32_t n, int32_t* added);
  int prefix_match(const int32_t* tokens, int32_t n, pkv_seq* out, int32_t* matched);
  void prefix_clear();
  int32_t prefix_entries() const { return n_ent_; }
  int32_t prefix_evictable() const;
  int set_prefix_capacity(int64_t cap);

  // Plans appends for seqs[i] += counts[i] tokens, in order, all or nothing.
  // Slots are appended to `slots` in (sequence, token) order; copies to `cows`.
  int append_plan_batch(const pkv_seq* seqs, const int32_t* counts, int32_t n,
                        std::vector<int64_t>* slots, std::vector<pkv_cow_op>* cows);

  int seq_info(pkv_seq s, int32_t* len, int32_t* nblk) const;
  int seq_blocks(pkv_seq s, int32_t* out, int32_t cap) const;
  // Sequences and prompt-cache entries holding a block (one pass over the
  // tables; for inspection, not for the hot path).
  int refcount(int32_t id, int32_t* rc) const;
  int refcounts(int32_t* out, int32_t n) const;
  int stats(pkv_stats* st) const;

  // Validates a handle; returns the sequence or nullptr (error set).
  const Seq* get(pkv_seq s) const;
  // The sequence's block ids in logical order.
  const std::vector<int32_t>& blocks(const Seq& s) const;
  uint64_t mutation() const { return mutation_; }

 private:
  Seq* get_mut(pkv_seq s);
  int32_t take_block();  // caller has checked availability (free or evictable)
  void release_ref(int32_t b);

  // persistent tables
  int32_t new_chunk();
  int32_t new_list();
  void drop_chunk(int32_t c);   // one reference less; at zero its blocks lose one
  void drop_list(int32_t l);    // one reference less; at zero its chunks lose one
  void own_list(Seq& s);        // s's list, copied first if shared (created if none)
  void own_last_chunk(Seq& s);  // s's last chunk, copied first if shared
  void push_id(Seq& s, int32_t b);     // appends block b (one more reference on it)
  void set_last_id(Seq& s, int32_t b); // replaces the last block id (no count change)
  void cut_table(Seq& s, int32_t keep);  // keeps the first `keep` block ids
  void effective_refs(std::vector<int32_t>& out) const;
#ifdef PKV_CHECKS
  void check_exclusive(const Seq& s, int32_t b) const;
#endif

  int32_t find_entry(int32_t parent, const int32_t* toks, uint64_t h) const;
  bool evict_one(uint64_t spare_stamp);  // false: nothing evictable
  void drop_entry(int32_t e);

  pkv_pool_desc d_;
  std::vector<int32_t> order_;    // rank -> block id
  std::vector<int32_t> rank_of_;  // block id -> rank
  std::vector<int32_t> ref_;
  FreeSet free_;
  std::vector<Seq> seqs_;
  std::vector<int32_t> free_seq_slots_;
  std::vector<TChunk> chunks_;
  std::vector<int32_t> free_chunks_;
  std::vector<TList> lists_;
  std::vector<int32_t> free_lists_;
  int32_t live_ = 0;
  uint64_t mutation_ = 0;  // bumped by every table change
  int64_t ids_copied_ = 0;  // block ids and chunk references copied (own_list, own_last_chunk)

  std::vector<CacheEntry> ents_;
  std::vector<int32_t> ent_tok_;  // block_size token ids per entry slot
  std::vector<int32_t> ent_free_;
  std::unordered_multimap<uint64_t, int32_t> ent_index_;
  int32_t n_ent_ = 0;
  int32_t cache_cap_ = 0;
  uint64_t clock_ = 0;
};

}  // namespace pkv
