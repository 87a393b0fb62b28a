// Host block pool, block tables, fork / free and the append planner.
// See pool.hpp for the mechanism and its source.
#include "pool.hpp"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <unordered_map>

namespace pkv {

namespace {

// Whether a sequence appears more than once in a batch (O(n log n)).
bool listed_twice(const pkv_seq* seqs, int32_t n) {
  std::vector<int32_t> idx((size_t)n);
  for (int32_t i = 0; i < n; ++i) idx[i] = seqs[i].index;
  std::sort(idx.begin(), idx.end());
  return std::adjacent_find(idx.begin(), idx.end()) != idx.end();
}
thread_local std::string g_err;
}

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}
void clear_error() { g_err.clear(); }
const char* last_error() { return g_err.c_str(); }

// ------------------------------------------------------------------ FreeSet

void FreeSet::init(int n) {
  n_ = n;
  count_ = n;
  lv_.clear();
  int bits = n;
  do {
    int words = (bits + 63) / 64;
    std::vector<uint64_t> w(words, ~0ull);
    if (bits % 64) w.back() = (1ull << (bits % 64)) - 1;
    lv_.push_back(std::move(w));
    bits = words;
  } while (bits > 1);
}

int FreeSet::pop_lowest() {
  if (count_ == 0) return -1;
  // descend from the top summary level
  int idx = 0;
  for (int k = (int)lv_.size() - 1; k >= 0; --k) {
    uint64_t w = lv_[k][idx];
    idx = idx * 64 + __builtin_ctzll(w);
  }
  int rank = idx;
  // clear the leaf bit and propagate emptiness upward
  int i = rank;
  for (size_t k = 0; k < lv_.size(); ++k) {
    uint64_t& w = lv_[k][i / 64];
    w &= ~(1ull << (i % 64));
    if (w != 0) break;
    i /= 64;
  }
  --count_;
  return rank;
}

void FreeSet::insert(int rank) {
  int i = rank;
  for (size_t k = 0; k < lv_.size(); ++k) {
    uint64_t& w = lv_[k][i / 64];
    bool was_empty = (w == 0);
    w |= 1ull << (i % 64);
    if (!was_empty) break;
    i /= 64;
  }
  ++count_;
}

void FreeSet::erase(int rank) {
  int i = rank;
  for (size_t k = 0; k < lv_.size(); ++k) {
    uint64_t& w = lv_[k][i / 64];
    w &= ~(1ull << (i % 64));
    if (w != 0) break;
    i /= 64;
  }
  --count_;
}

bool FreeSet::contains(int rank) const { return (lv_[0][rank / 64] >> (rank % 64)) & 1ull; }

// --------------------------------------------------------------------- Pool

Pool::Pool(const pkv_pool_desc& d) : d_(d) {
  const int nb = d.num_blocks;
  order_.resize(nb);
  rank_of_.resize(nb);
  for (int i = 0; i < nb; ++i) order_[i] = d.alloc_order ? d.alloc_order[i] : i;
  for (int i = 0; i < nb; ++i) rank_of_[order_[i]] = i;
  d_.alloc_order = nullptr;  // copied; do not keep the caller's pointer
  ref_.assign(nb, 0);
  free_.init(nb);
  cache_cap_ = nb;
}

void Pool::release_ref(int32_t b) {
  if (--ref_[b] == 0) free_.insert(rank_of_[b]);
}

int32_t Pool::take_block() {
  if (free_.count() == 0) evict_one(0);
  int rank = free_.pop_lowest();
  int32_t b = order_[rank];
  ref_[b] = 1;
  return b;
}

int Pool::block_alloc(int32_t* id) {
  if (!id) return fail(PKV_E_INVALID, "block_alloc: null output");
  if (free_.count() == 0 && !evict_one(0)) return fail(PKV_E_OOM, "block_alloc: pool exhausted");
  *id = take_block();
  ++mutation_;
  return PKV_OK;
}

int Pool::block_release(int32_t id) {
  if (id < 0 || id >= d_.num_blocks) return fail(PKV_E_INVALID, "block_release: id out of range");
  if (ref_[id] <= 0) return fail(PKV_E_INVALID, "block_release: block is already free");
  release_ref(id);
  ++mutation_;
  return PKV_OK;
}

const Seq* Pool::get(pkv_seq s) const {
  if (s.index < 0 || s.index >= (int32_t)seqs_.size() || !seqs_[s.index].live ||
      seqs_[s.index].gen != s.generation) {
    fail(PKV_E_INVALID, "invalid or stale sequence handle");
    return nullptr;
  }
  return &seqs_[s.index];
}

Seq* Pool::get_mut(pkv_seq s) { return const_cast<Seq*>(get(s)); }

// ------------------------------------------------------ persistent tables

int32_t Pool::new_chunk() {
  int32_t c;
  if (!free_chunks_.empty()) {
    c = free_chunks_.back();
    free_chunks_.pop_back();
  } else {
    c = (int32_t)chunks_.size();
    chunks_.emplace_back();
  }
  chunks_[c].ref = 1;
  chunks_[c].n = 0;
  return c;
}

int32_t Pool::new_list() {
  int32_t l;
  if (!free_lists_.empty()) {
    l = free_lists_.back();
    free_lists_.pop_back();
  } else {
    l = (int32_t)lists_.size();
    lists_.emplace_back();
  }
  lists_[l].ref = 1;
  lists_[l].chunks.clear();
  return l;
}

void Pool::drop_chunk(int32_t c) {
  TChunk& k = chunks_[c];
  if (--k.ref > 0) return;
  for (int32_t i = 0; i < k.n; ++i) release_ref(k.ids[i]);
  k.n = 0;
  free_chunks_.push_back(c);
}

void Pool::drop_list(int32_t l) {
  if (--lists_[l].ref > 0) return;
  for (int32_t c : lists_[l].chunks) drop_chunk(c);
  lists_[l].chunks.clear();
  free_lists_.push_back(l);
}

void Pool::own_list(Seq& s) {
  if (s.list < 0) {
    s.list = new_list();
    return;
  }
  if (lists_[s.list].ref == 1) return;
  const int32_t old = s.list;
  const int32_t l = new_list();  // (may reallocate lists_)
  lists_[l].chunks = lists_[old].chunks;
  for (int32_t c : lists_[l].chunks) ++chunks_[c].ref;
  ids_copied_ += (int64_t)lists_[l].chunks.size();
  --lists_[old].ref;  // still held by the sequences that shared it
  s.list = l;
}

void Pool::own_last_chunk(Seq& s) {
  std::vector<int32_t>& cl = lists_[s.list].chunks;
  const int32_t old = cl.back();
  if (chunks_[old].ref == 1) return;
  const int32_t c = new_chunk();  // (may reallocate chunks_)
  TChunk& k = chunks_[c];
  const TChunk& o = chunks_[old];
  k.n = o.n;
  for (int32_t i = 0; i < o.n; ++i) {
    k.ids[i] = o.ids[i];
    ++ref_[o.ids[i]];
  }
  ids_copied_ += o.n;
  --chunks_[old].ref;  // still held by the lists that shared it
  lists_[s.list].chunks.back() = c;
}

void Pool::push_id(Seq& s, int32_t b) {
  own_list(s);
  std::vector<int32_t>& cl = lists_[s.list].chunks;
  if (cl.empty() || chunks_[cl.back()].n == kChunk) {
    const int32_t c = new_chunk();
    lists_[s.list].chunks.push_back(c);
  } else {
    own_last_chunk(s);
  }
  TChunk& k = chunks_[lists_[s.list].chunks.back()];
  k.ids[k.n++] = b;
  s.flat_ok = false;
}

void Pool::set_last_id(Seq& s, int32_t b) {
  own_list(s);
  own_last_chunk(s);
  TChunk& k = chunks_[lists_[s.list].chunks.back()];
  k.ids[k.n - 1] = b;
  s.flat_ok = false;
}

void Pool::cut_table(Seq& s, int32_t keep) {
  if (s.list < 0) return;
  const int32_t have = (int32_t)((s.len + (int64_t)d_.block_size - 1) / d_.block_size);
  if (keep >= have) return;
  s.flat_ok = false;
  if (keep == 0) {
    drop_list(s.list);
    s.list = -1;
    return;
  }
  own_list(s);
  std::vector<int32_t>& cl = lists_[s.list].chunks;
  const int32_t keep_chunks = (keep + kChunk - 1) / kChunk;
  while ((int32_t)cl.size() > keep_chunks) {
    const int32_t c = cl.back();
    cl.pop_back();
    drop_chunk(c);
  }
  const int32_t in_last = keep - (keep_chunks - 1) * kChunk;
  if (chunks_[cl.back()].n > in_last) {
    own_last_chunk(s);
    TChunk& k = chunks_[lists_[s.list].chunks.back()];
    for (int32_t i = in_last; i < k.n; ++i) release_ref(k.ids[i]);
    k.n = in_last;
  }
}

const std::vector<int32_t>& Pool::blocks(const Seq& s) const {
  if (!s.flat_ok) {
    s.flat.clear();
    if (s.list >= 0)
      for (int32_t c : lists_[s.list].chunks)
        s.flat.insert(s.flat.end(), chunks_[c].ids, chunks_[c].ids + chunks_[c].n);
    s.flat_ok = true;
  }
  return s.flat;
}

void Pool::effective_refs(std::vector<int32_t>& out) const {
  // a chunk stands for as many holders as the sequences of the lists that
  // hold it; ref_ counts it once
  out.assign(ref_.begin(), ref_.end());
  std::vector<int64_t> w(chunks_.size(), 0);
  for (const TList& l : lists_)
    if (l.ref > 0)
      for (int32_t c : l.chunks) w[c] += l.ref;
  for (size_t c = 0; c < chunks_.size(); ++c) {
    const TChunk& k = chunks_[c];
    if (k.ref <= 0) continue;
    for (int32_t i = 0; i < k.n; ++i) out[k.ids[i]] += (int32_t)(w[c] - 1);
  }
}

// -------------------------------------------------------------- sequences

int Pool::seq_create(pkv_seq* out) {
  if (!out) return fail(PKV_E_INVALID, "seq_create: null output");
  int32_t idx;
  if (!free_seq_slots_.empty()) {
    idx = free_seq_slots_.back();
    free_seq_slots_.pop_back();
  } else {
    idx = (int32_t)seqs_.size();
    seqs_.emplace_back();
  }
  Seq& s = seqs_[idx];
  s.live = true;
  s.len = 0;
  s.list = -1;
  s.flat.clear();
  s.flat_ok = true;
  ++live_;
  ++mutation_;
  *out = pkv_seq{idx, s.gen};
  return PKV_OK;
}

int Pool::seq_fork(pkv_seq parent, pkv_seq* child) {
  if (!child) return fail(PKV_E_INVALID, "seq_fork: null output");
  if (!get(parent)) return PKV_E_INVALID;
  pkv_seq c;
  int rc = seq_create(&c);  // may grow seqs_: re-fetch the parent after
  if (rc) return rc;
  const Seq& p = seqs_[parent.index];
  Seq& k = seqs_[c.index];
  k.list = p.list;  // shared: one count, whatever the table's length
  if (k.list >= 0) ++lists_[k.list].ref;
  k.len = p.len;
  k.flat_ok = false;
  *child = c;
  return PKV_OK;
}

int Pool::seq_free(pkv_seq h) {
  Seq* s = get_mut(h);
  if (!s) return PKV_E_INVALID;
  if (s->list >= 0) drop_list(s->list);
  s->list = -1;
  s->flat.clear();
  s->flat_ok = true;
  s->len = 0;
  s->live = false;
  ++s->gen;
  free_seq_slots_.push_back(h.index);
  --live_;
  ++mutation_;
  return PKV_OK;
}

int Pool::seq_truncate(pkv_seq h, int32_t n) {
  Seq* s = get_mut(h);
  if (!s) return PKV_E_INVALID;
  if (n < 0 || n > s->len) return fail(PKV_E_INVALID, "truncate: length outside [0, len]");
  cut_table(*s, (int32_t)((n + (int64_t)d_.block_size - 1) / d_.block_size));
  s->len = n;
  ++mutation_;
  return PKV_OK;
}

int Pool::truncate_append(pkv_seq h, int32_t keep_len, int32_t n_new, std::vector<int64_t>* slots,
                          std::vector<pkv_cow_op>* cows) {
  return truncate_append_batch(&h, &keep_len, &n_new, 1, slots, cows);
}

int Pool::truncate_append_batch(const pkv_seq* seqs, const int32_t* keep_lens, const int32_t* n_new,
                                int32_t n, std::vector<int64_t>* slots,
                                std::vector<pkv_cow_op>* cows) {
  if (n < 0 || (n > 0 && (!seqs || !keep_lens || !n_new)))
    return fail(PKV_E_INVALID, "truncate_append: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = get(seqs[i]);
    if (!s) return PKV_E_INVALID;
    if (keep_lens[i] < 0 || keep_lens[i] > s->len)
      return fail(PKV_E_INVALID, "truncate: length outside [0, len]");
  }
  if (listed_twice(seqs, n)) return fail(PKV_E_INVALID, "truncate_append: a sequence appears twice");
  std::vector<std::vector<int32_t>> tails((size_t)n);
  std::vector<int32_t> old_len((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = seqs_[seqs[i].index];
    old_len[i] = s.len;
    const int32_t keep = (int32_t)((keep_lens[i] + (int64_t)d_.block_size - 1) / d_.block_size);
    const std::vector<int32_t>& all = blocks(s);
    tails[i].assign(all.begin() + keep, all.end());
    seq_truncate(seqs[i], keep_lens[i]);
  }
  int rc = append_plan_batch(seqs, n_new, n, slots, cows);
  if (rc == PKV_OK) return rc;
  // the refused append changed nothing a caller sees: give the tails back
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = seqs_[seqs[i].index];
    for (int32_t b : tails[i]) {
      if (ref_[b] == 0) free_.erase(rank_of_[b]);
      ++ref_[b];
      push_id(s, b);
    }
    s.len = old_len[i];
  }
  return rc;
}

int Pool::append_plan_batch(const pkv_seq* seqs, const int32_t* counts, int32_t n,
                            std::vector<int64_t>* slots, std::vector<pkv_cow_op>* cows) {
  if (n < 0 || (n > 0 && (!seqs || !counts))) return fail(PKV_E_INVALID, "append: bad arguments");
  const int64_t bs = d_.block_size;
  // Pass 0: validate.
  if (listed_twice(seqs, n)) return fail(PKV_E_INVALID, "append: a sequence appears twice in one batch");
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = get(seqs[i]);
    if (!s) return PKV_E_INVALID;
    if (counts[i] < 0) return fail(PKV_E_INVALID, "append: negative token count");
    if ((int64_t)s->len + counts[i] > (int64_t)INT32_MAX)
      return fail(PKV_E_INVALID, "append: sequence length overflow");
  }
  // Pass 1: give every appending sequence its own list and, where the tail
  // block is partly filled, its own last chunk (copies of shared table
  // parts change nothing a caller sees and allocate no block), so that a
  // tail block's count is the number of its holders' chunks. Then count
  // the blocks the batch needs in the order pass 2 takes (a copy made by an
  // earlier sequence lowers the count of a tail that a later one shares).
  for (int32_t i = 0; i < n; ++i) {
    if (counts[i] == 0) continue;
    Seq& s = seqs_[seqs[i].index];
    own_list(s);
    if (s.len % bs != 0) own_last_chunk(s);
  }
  std::unordered_map<int32_t, int32_t> dropped;  // block -> refs dropped by earlier copies
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (counts[i] == 0) continue;
    const Seq& s = seqs_[seqs[i].index];
    if (s.len % bs != 0) {
      const TChunk& k = chunks_[lists_[s.list].chunks.back()];
      const int32_t last = k.ids[k.n - 1];
      if (ref_[last] - dropped[last] > 1) {
        ++need;
        ++dropped[last];
      }
    }
    int64_t before = (s.len + bs - 1) / bs, after = (s.len + counts[i] + bs - 1) / bs;
    need += after - before;
  }
  if (need > free_.count() && need > (int64_t)free_.count() + prefix_evictable())
    return fail(PKV_E_OOM, "append: pool has " + std::to_string(free_.count()) +
                               " free blocks, the append needs " + std::to_string(need));
  // Pass 2: execute (cannot fail).
  for (int32_t i = 0; i < n; ++i) {
    if (counts[i] == 0) continue;
    Seq& s = seqs_[seqs[i].index];
    const int32_t r = (int32_t)(s.len % bs);
    if (r != 0) {
      const TChunk& k = chunks_[lists_[s.list].chunks.back()];
      const int32_t old = k.ids[k.n - 1];
      if (ref_[old] > 1) {
        const int32_t fresh = take_block();
        --ref_[old];  // (> 0: another chunk or entry still holds it)
        set_last_id(s, fresh);
        if (cows) cows->push_back(pkv_cow_op{old, fresh, r});
      }
    }
    int32_t cur = -1;
    for (int32_t t = 0; t < counts[i]; ++t) {
      const int64_t pos = s.len;
      if (pos % bs == 0) {
        cur = take_block();
        push_id(s, cur);
      } else if (cur < 0) {
        const TChunk& k = chunks_[lists_[s.list].chunks.back()];
        cur = k.ids[k.n - 1];
      }
#ifdef PKV_CHECKS
      check_exclusive(s, cur);
#endif
      if (slots) slots->push_back((int64_t)cur * bs + pos % bs);
      ++s.len;
    }
    s.flat_ok = false;
  }
  if (need || n) ++mutation_;
  return PKV_OK;
}

#ifdef PKV_CHECKS
// Debug builds (build.py --sanitize): a block about to be written must have
// exactly one holder ([D2]: a block being written is never aliased): its
// count is 1 and the table list and chunk through which the writer holds it
// are the writer's alone. Aborts otherwise.
void Pool::check_exclusive(const Seq& s, int32_t b) const {
  const TList& l = lists_[s.list];
  const TChunk& k = chunks_[l.chunks.back()];
  if (ref_[b] != 1 || l.ref != 1 || k.ref != 1 || k.n == 0 || k.ids[k.n - 1] != b) {
    std::fprintf(stderr, "pkv: write into shared block %d (count %d, list %d, chunk %d)\n", b,
                 ref_[b], l.ref, k.ref);
    std::abort();
  }
}
#endif

// ------------------------------------------------------------ prompt cache

namespace {
uint64_t key_hash(int32_t parent, const int32_t* toks, int n) {
  uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)(uint32_t)parent;
  for (int i = 0; i < n; ++i) {
    h ^= (uint64_t)(uint32_t)toks[i] + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
    h *= 0xFF51AFD7ED558CCDull;
  }
  return h ^ (h >> 33);
}
}  // namespace

int32_t Pool::find_entry(int32_t parent, const int32_t* toks, uint64_t h) const {
  const int bs = d_.block_size;
  auto range = ent_index_.equal_range(h);
  for (auto it = range.first; it != range.second; ++it) {
    const int32_t e = it->second;
    if (ents_[e].parent == parent &&
        std::equal(toks, toks + bs, ent_tok_.begin() + (size_t)e * bs))
      return e;
  }
  return -1;
}

bool Pool::evict_one(uint64_t spare_stamp) {
  int32_t best = -1;
  for (int32_t e = 0; e < (int32_t)ents_.size(); ++e) {
    const CacheEntry& r = ents_[e];
    if (!r.live || r.n_child || ref_[r.block] != 1 || r.stamp == spare_stamp) continue;
    if (best < 0 || r.stamp < ents_[best].stamp ||
        (r.stamp == ents_[best].stamp && r.depth > ents_[best].depth))
      best = e;
  }
  if (best < 0) return false;
  drop_entry(best);
  return true;
}

void Pool::drop_entry(int32_t e) {
  CacheEntry& r = ents_[e];
  auto range = ent_index_.equal_range(r.hash);
  for (auto it = range.first; it != range.second; ++it)
    if (it->second == e) {
      ent_index_.erase(it);
      break;
    }
  if (r.parent >= 0) --ents_[r.parent].n_child;
  release_ref(r.block);
  r.live = false;
  ent_free_.push_back(e);
  --n_ent_;
  ++mutation_;
}

int32_t Pool::prefix_evictable() const {
  if (n_ent_ == 0) return 0;
  // an entry can go once its whole subtree can: visit children before parents
  std::vector<int32_t> ids;
  ids.reserve((size_t)n_ent_);
  for (int32_t e = 0; e < (int32_t)ents_.size(); ++e)
    if (ents_[e].live) ids.push_back(e);
  std::sort(ids.begin(), ids.end(),
            [&](int32_t a, int32_t b) { return ents_[a].depth > ents_[b].depth; });
  std::vector<uint8_t> blocked(ents_.size(), 0);
  int32_t n = 0;
  for (int32_t e : ids) {
    const CacheEntry& r = ents_[e];
    const bool ok = !blocked[e] && ref_[r.block] == 1;
    if (ok)
      ++n;
    else if (r.parent >= 0)
      blocked[r.parent] = 1;
  }
  return n;
}

int Pool::prefix_insert(pkv_seq h, const int32_t* tokens, int32_t n, int32_t* added) {
  const Seq* s = get(h);
  if (!s) return PKV_E_INVALID;
  if (n < 0 || (n > 0 && !tokens)) return fail(PKV_E_INVALID, "prefix_insert: bad token list");
  if (n > s->len) return fail(PKV_E_INVALID, "prefix_insert: more token ids than the sequence holds");
  const int bs = d_.block_size;
  const uint64_t stamp = ++clock_;
  int32_t parent = -1, count = 0;
  for (int32_t i = 0; i < n / bs; ++i) {
    const int32_t* t = tokens + (size_t)i * bs;
    const uint64_t hk = key_hash(parent, t, bs);
    int32_t e = find_entry(parent, t, hk);
    if (e >= 0) {
      ents_[e].stamp = stamp;
      parent = e;
      continue;
    }
    if (n_ent_ >= cache_cap_ && !evict_one(stamp)) break;
    if (!ent_free_.empty()) {
      e = ent_free_.back();
      ent_free_.pop_back();
    } else {
      e = (int32_t)ents_.size();
      ents_.emplace_back();
      ent_tok_.resize(ents_.size() * (size_t)bs);
    }
    CacheEntry& r = ents_[e];
    r.parent = parent;
    r.block = blocks(*s)[(size_t)i];
    r.depth = parent < 0 ? 1 : ents_[parent].depth + 1;
    r.n_child = 0;
    r.stamp = stamp;
    r.hash = hk;
    r.live = true;
    std::copy(t, t + bs, ent_tok_.begin() + (size_t)e * bs);
    if (parent >= 0) ++ents_[parent].n_child;
    ent_index_.emplace(hk, e);
    ++ref_[r.block];
    ++n_ent_;
    parent = e;
    ++count;
  }
  if (count) ++mutation_;
  if (added) *added = count;
  return PKV_OK;
}

int Pool::prefix_match(const int32_t* tokens, int32_t n, pkv_seq* out, int32_t* matched) {
  if (!out) return fail(PKV_E_INVALID, "prefix_match: null output");
  if (n < 0 || (n > 0 && !tokens)) return fail(PKV_E_INVALID, "prefix_match: bad token list");
  const int bs = d_.block_size;
  const uint64_t stamp = ++clock_;
  std::vector<int32_t> chain;
  int32_t parent = -1;
  for (int32_t i = 0; i < n / bs; ++i) {
    const int32_t* t = tokens + (size_t)i * bs;
    const int32_t e = find_entry(parent, t, key_hash(parent, t, bs));
    if (e < 0) break;
    ents_[e].stamp = stamp;
    chain.push_back(e);
    parent = e;
  }
  pkv_seq c;
  int rc = seq_create(&c);
  if (rc) return rc;
  Seq& k = seqs_[c.index];
  for (int32_t e : chain) {
    ++ref_[ents_[e].block];
    push_id(k, ents_[e].block);
  }
  k.len = (int32_t)chain.size() * bs;
  *out = c;
  if (matched) *matched = k.len;
  return PKV_OK;
}

void Pool::prefix_clear() {
  for (int32_t e = 0; e < (int32_t)ents_.size(); ++e)
    if (ents_[e].live) release_ref(ents_[e].block);
  ents_.clear();
  ent_tok_.clear();
  ent_free_.clear();
  ent_index_.clear();
  n_ent_ = 0;
  ++mutation_;
}

int Pool::set_prefix_capacity(int64_t cap) {
  if (cap < 0 || cap > d_.num_blocks)
    return fail(PKV_E_INVALID, "prefix cache capacity outside [0, num_blocks]");
  cache_cap_ = (int32_t)cap;
  return PKV_OK;
}

int Pool::seq_info(pkv_seq h, int32_t* len, int32_t* nblk) const {
  const Seq* s = get(h);
  if (!s) return PKV_E_INVALID;
  if (len) *len = s->len;
  if (nblk) *nblk = (int32_t)((s->len + (int64_t)d_.block_size - 1) / d_.block_size);
  return PKV_OK;
}

int Pool::seq_blocks(pkv_seq h, int32_t* out, int32_t cap) const {
  const Seq* s = get(h);
  if (!s) return PKV_E_INVALID;
  if (cap < 0 || (cap > 0 && !out)) return fail(PKV_E_INVALID, "seq_blocks: bad buffer");
  const std::vector<int32_t>& t = blocks(*s);
  int32_t m = std::min<int32_t>(cap, (int32_t)t.size());
  std::copy(t.begin(), t.begin() + m, out);
  return PKV_OK;
}

int Pool::refcount(int32_t id, int32_t* rc) const {
  if (id < 0 || id >= d_.num_blocks || !rc) return fail(PKV_E_INVALID, "refcount: bad block id");
  std::vector<int32_t> all;
  effective_refs(all);
  *rc = all[id];
  return PKV_OK;
}

int Pool::refcounts(int32_t* out, int32_t n) const {
  if (n < 0 || n > d_.num_blocks || (n > 0 && !out)) return fail(PKV_E_INVALID, "refcounts: bad buffer");
  std::vector<int32_t> all;
  effective_refs(all);
  std::copy(all.begin(), all.begin() + n, out);
  return PKV_OK;
}

int Pool::stats(pkv_stats* st) const {
  if (!st) return fail(PKV_E_INVALID, "stats: null output");
  st->num_blocks = d_.num_blocks;
  st->free_blocks = free_.count();
  st->live_seqs = live_;
  st->reserved = 0;
  // (sequences, prompt-cache entries and blocks taken with block_alloc)
  std::vector<int32_t> all;
  effective_refs(all);
  int64_t refs = 0;
  for (int32_t r : all) refs += r;
  st->total_refs = refs;
  st->table_ids_copied = ids_copied_;
  return PKV_OK;
}

}  // namespace pkv
