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
  bool contains(int rank) const;

 private:
  std::vector<std::vector<uint64_t>> lv_;  // lv_[0] leaf bits, lv_[k+1] = nonzero words of lv_[k]
  int n_ = 0;
  int count_ = 0;
};

struct Seq {
  uint32_t gen = 1;
  bool live = false;
  int32_t len = 0;
  std::vector<int32_t> blocks;
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

  // Plans appends for seqs[i] += counts[i] tokens, in order, all or nothing.
  // Slots are appended to `slots` in (sequence, token) order; copies to `cows`.
  int append_plan_batch(const pkv_seq* seqs, const int32_t* counts, int32_t n,
                        std::vector<int64_t>* slots, std::vector<pkv_cow_op>* cows);

  int seq_info(pkv_seq s, int32_t* len, int32_t* nblk) const;
  int seq_blocks(pkv_seq s, int32_t* out, int32_t cap) const;
  int refcount(int32_t id, int32_t* rc) const;
  int stats(pkv_stats* st) const;

  // Validates a handle; returns the sequence or nullptr (error set).
  const Seq* get(pkv_seq s) const;
  uint64_t mutation() const { return mutation_; }

 private:
  Seq* get_mut(pkv_seq s);
  int32_t take_block();  // caller has checked availability

  pkv_pool_desc d_;
  std::vector<int32_t> order_;    // rank -> block id
  std::vector<int32_t> rank_of_;  // block id -> rank
  std::vector<int32_t> ref_;
  FreeSet free_;
  std::vector<Seq> seqs_;
  std::vector<int32_t> free_seq_slots_;
  int32_t live_ = 0;
  int64_t total_refs_ = 0;
  uint64_t mutation_ = 0;  // bumped by every table change
};

}  // namespace pkv
