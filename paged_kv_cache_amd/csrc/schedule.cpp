// Attention planner: segments, chunks, work items and combine lists.
//
// Sharing comes from forks, which copy a table prefix; so two sequences that
// hold the same block hold it at the same logical position, and the blocks a
// set of sequences shares form a common prefix of each of their tables.
// Grouping consecutive blocks by their holder set therefore cuts the batch
// into a tree of segments; each segment's K/V is read by one set of work
// items and applied to every row (holder x query head) that needs it.
#include "schedule.hpp"

#include <algorithm>
#include <stdexcept>
#include <cstring>
#include <unordered_map>

namespace pkv {

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int32_t round_up(int32_t x, int32_t m) { return (x + m - 1) / m * m; }

struct Segment {
  std::vector<int32_t> blocks;  // logical order
  int32_t t0 = 0;               // logical position of the first token
  int32_t n_tok = 0;
  int32_t hold_off = 0;         // into Schedule::holders
  int32_t n_hold = 0;
  int32_t chunk_begin = 0, chunk_end = 0;  // into the chunk list
  int32_t mask_from = 0x7fffffff;          // draft-tree mask start (verify)
  // a group of branches (see group_runs): per block, the holder bits and
  // valid slots (<< 16); n_tok is then blocks * block size
  std::vector<int32_t> binfo;
  int32_t all_bits = 0;                    // holder bits of all its holders
};

struct Chunk {
  int32_t seg;
  int32_t blk_off, n_tok, t0, part_base;
};

// Step granularity of the attention kernels, in tokens and in blocks.
int32_t step_tokens(int32_t bs) { return bs > 32 ? bs : 32; }

// Cuts every segment into chunks and every chunk's rows into work items.
std::vector<Chunk> emit_chunks(std::vector<Segment>& segs, int32_t bs, int32_t G, int32_t n_layers,
                               int32_t Hkv, const SchedOptions& opt, Schedule* S) {
  const int32_t step = step_tokens(bs);
  const int32_t step_blocks = step / bs;
  const int32_t rpi = std::max<int32_t>(1, opt.rows_per_item);
  // chunk length per segment: long enough that the partial states a chunk
  // writes stay small next to the K/V it reads (rows * (D + 2) floats vs
  // tokens * 2 * D elements), short enough to fill the machine
  // no chunk spans more than kMaxChunkBlocks blocks
  const int32_t cap = (kMaxChunkBlocks / step_blocks) * step;
  const int32_t min_chunk = opt.min_chunk_tokens > 0 ? opt.min_chunk_tokens : 1024;
  const int32_t per_row = opt.tokens_per_row > 0 ? opt.tokens_per_row : 64;
  auto base_len = [&](const Segment& s) {
    if (opt.chunk_tokens > 0) return std::min(round_up(opt.chunk_tokens, step), cap);
    int32_t rows = s.n_hold * G;
    int32_t t = round_up(std::max(min_chunk, per_row * rows), step);
    return std::min({t, round_up(opt.max_chunk_tokens, step), cap});
  };
  auto count_wgs = [&](int32_t div) {
    int64_t w = 0;
    for (const Segment& s : segs) {
      int32_t len =
          std::min(cap, std::max(round_up(min_chunk, step), round_up(base_len(s) / div, step)));
      if (opt.chunk_tokens > 0) len = base_len(s);
      int64_t chunks = (s.n_tok + len - 1) / len;
      const int64_t rows = (int64_t)s.n_hold * G;
      int64_t items = (opt.wide && rows > rpi) ? (rows + opt.wide_rows - 1) / opt.wide_rows
                                               : (rows + rpi - 1) / rpi;
      w += chunks * items;
    }
    return w * n_layers * Hkv;
  };
  int32_t div = 1;
  if (opt.chunk_tokens <= 0) {
    // (three quarters: one workgroup per CU on 3/4 of the chip beats two
    // half-length rounds on all of it plus twice the partial states)
    while (div < 64 && 4 * count_wgs(div) < 3 * (int64_t)opt.target_workgroups &&
           count_wgs(div * 2) > count_wgs(div))
      div *= 2;
  }
  std::vector<Chunk> chunks;
  for (size_t si = 0; si < segs.size(); ++si) {
    Segment& s = segs[si];
    int32_t len = opt.chunk_tokens > 0
                      ? base_len(s)
                      : std::min(cap, std::max(round_up(min_chunk, step),
                                               round_up(base_len(s) / div, step)));
    const int32_t nb = (int32_t)s.blocks.size();
    int32_t k = (s.n_tok + len - 1) / len;
    // equal chunks of whole steps
    int32_t per = round_up((nb + k - 1) / k, step_blocks);
    if (per > kMaxChunkBlocks) throw std::logic_error("planner: chunk longer than kMaxChunkBlocks");
    s.chunk_begin = (int32_t)chunks.size();
    for (int32_t b0 = 0; b0 < nb; b0 += per) {
      int32_t b1 = std::min(nb, b0 + per);
      Chunk c;
      c.seg = (int32_t)si;
      c.blk_off = (int32_t)S->blk.size();
      c.t0 = s.t0 + b0 * bs;
      c.n_tok = std::min(s.n_tok, (b1 - b0) * bs + b0 * bs) - b0 * bs;
      for (int32_t b = b0; b < b1; ++b) S->blk.push_back(s.blocks[b]);
      while ((S->blk.size() - c.blk_off) % step_blocks) S->blk.push_back(s.blocks[b1 - 1]);
      if (S->grouped) {
        for (int32_t b = b0; b < b1; ++b) S->binfo.push_back(s.binfo.empty() ? 0 : s.binfo[b]);
        S->binfo.resize(S->blk.size(), 0);  // padding: no holder, no valid slot
      }
      c.part_base = S->P;
      S->P += s.n_hold * G;
      chunks.push_back(c);
    }
    s.chunk_end = (int32_t)chunks.size();
  }
  S->n_chunks = (int32_t)chunks.size();
  // narrow items: up to rpi rows; wide items (more rows than that): the
  // rows split evenly in whole 16-row blocks, at most wide_rows each
  std::vector<WorkItem> narrow;
  std::vector<std::vector<WorkItem>> wide_groups;
  for (const Chunk& c : chunks) {
    const Segment& s = segs[c.seg];
    const int32_t rows = s.n_hold * G;
    WorkItem w{};
    w.blk_off = c.blk_off;
    w.n_tok = c.n_tok;
    w.t0 = c.t0;
    w.hold_off = s.hold_off;
    w.mask_from = s.mask_from;
    w.grouped = s.all_bits;
    if (s.all_bits && rows > rpi) throw std::logic_error("planner: a grouped item wider than a narrow one");
    if (opt.wide && rows > rpi) {
      S->wide_tokens += c.n_tok;
      // wide items of one chunk (siblings) read it through the shared L2
      // (rows split evenly in whole blocks, or with wide_fill every item
      // but the last full)
      const int32_t k = (rows + opt.wide_rows - 1) / opt.wide_rows;
      const int32_t per = opt.wide_fill ? std::max<int32_t>(16, opt.wide_rows / 16 * 16)
                                        : round_up((rows + k - 1) / k, 16);
      std::vector<WorkItem> grp;
      w.reread = per < rows ? 1 : 0;
      for (int32_t r0 = 0; r0 < rows; r0 += per) {
        w.r0 = r0;
        w.n_rows = std::min(per, rows - r0);
        w.part_row = c.part_base + r0;
        grp.push_back(w);
      }
      wide_groups.push_back(std::move(grp));
    } else {
      // several items of one chunk each read it (the rows of one item
      // more than one wave owns are marked below)
      for (int32_t r0 = 0; r0 < rows; r0 += rpi) {
        w.r0 = r0;
        w.n_rows = std::min(rpi, rows - r0);
        w.part_row = c.part_base + r0;
        w.reread = rpi < rows ? 1 : 0;
        narrow.push_back(w);
      }
    }
  }
  // a narrow wave owns two 16-row blocks when some item has more than 16
  // rows (and the head size leaves the registers for it); an item with
  // more rows than one wave owns has several waves loading each step
  // (automatic: only when such items carry a good share of the bytes, since
  // two blocks per wave cost every item of the launch an occupancy step)
  int32_t max_rows = 0;
  int64_t tok_all = 0, tok_big = 0;
  for (const WorkItem& w : narrow) {
    max_rows = std::max(max_rows, w.n_rows);
    tok_all += w.n_tok;
    tok_big += w.n_rows > 16 ? w.n_tok : 0;
  }
  const bool two = opt.max_row_blocks_per_wave == 2 ||
                   (opt.max_row_blocks_per_wave == 0 && 4 * tok_big >= tok_all);
  S->narrow_rw = (max_rows > 16 && two) ? 2 : 1;
  for (WorkItem& w : narrow)
    if (w.n_rows > 16 * S->narrow_rw) w.reread = 1;
  // longest chunks first, so the tail of each grid holds the short ones
  // (short items, one wave each, last); wide groups also by sibling count,
  // so equal counts sit together
  auto is_short = [&](const WorkItem& w) {
    return opt.short_items && w.n_rows <= 16 && w.n_tok <= opt.short_tokens;
  };
  std::stable_sort(narrow.begin(), narrow.end(), [&](const WorkItem& a, const WorkItem& b) {
    const bool sa = is_short(a), sb = is_short(b);
    if (sa != sb) return sb;  // long before short
    return a.n_tok > b.n_tok;
  });
  S->n_short = 0;
  for (const WorkItem& w : narrow) S->n_short += is_short(w) ? 1 : 0;
  S->long_by_plane = S->folded && opt.short_items;
  std::stable_sort(wide_groups.begin(), wide_groups.end(),
                   [](const std::vector<WorkItem>& a, const std::vector<WorkItem>& b) {
                     if (a.size() != b.size()) return a.size() > b.size();
                     return a[0].n_tok > b[0].n_tok;
                   });
  S->items = std::move(narrow);
  S->n_narrow = (int32_t)S->items.size();
  for (const auto& grp : wide_groups) S->items.insert(S->items.end(), grp.begin(), grp.end());
  S->build_order(n_layers, Hkv);
  return chunks;
}

// The tree plan: one item holding all n * G rows (row r = branch r / G,
// q-head offset r % G), every segment one or more chunks read once with the
// mask of the rows whose branch holds it. Segments of at least 64 rows (the
// shared root of a wide tree: matrix-core work) are cut into pieces of
// piece tokens and spread evenly, by tokens, among the other segments (the
// edges: memory traffic), so that a workgroup alternates between the two.
// Returns false (S untouched) if the batch does not fit the tree kernel.
bool plan_tree(const std::vector<Segment>& segs, int32_t n, int32_t bs, int32_t G,
               int32_t piece, Schedule* S) {
  const int32_t rows = n * G;
  if (rows > kTreeRows || rows <= 0) return false;
  struct Piece {
    int32_t seg, b0, b1, t0, n_tok;
  };
  std::vector<Piece> heavy, light;
  const int32_t unit = std::max<int32_t>(32, bs);           // whole steps and whole blocks
  const int32_t pblocks = std::max<int32_t>(1, round_up(std::max(piece, unit), unit) / bs);
  int64_t h_tok = 0, l_tok = 0;
  for (size_t k = 0; k < segs.size(); ++k) {
    const Segment& sg = segs[k];
    const int32_t nb = (int32_t)sg.blocks.size();
    const bool big = sg.n_hold * G >= 64;
    const int32_t step = big ? pblocks : nb;
    for (int32_t b0 = 0; b0 < nb; b0 += step) {
      const int32_t b1 = std::min(nb, b0 + step);
      Piece pc{(int32_t)k, b0, b1, sg.t0 + b0 * bs, std::min(sg.n_tok - b0 * bs, (b1 - b0) * bs)};
      (big ? heavy : light).push_back(pc);
      (big ? h_tok : l_tok) += pc.n_tok;
    }
  }
  if ((int64_t)heavy.size() + (int64_t)light.size() > kMaxTreeChunks) return false;
  // interleave by tokens: take the list that is behind its share
  std::vector<Piece> order;
  size_t hi = 0, li = 0;
  int64_t hd = 0, ld = 0;
  while (hi < heavy.size() || li < light.size()) {
    const bool take_h = li >= light.size() ||
                        (hi < heavy.size() && (double)hd * (double)std::max<int64_t>(l_tok, 1) <=
                                                  (double)ld * (double)std::max<int64_t>(h_tok, 1));
    if (take_h) {
      hd += heavy[hi].n_tok;
      order.push_back(heavy[hi++]);
    } else {
      ld += light[li].n_tok;
      order.push_back(light[li++]);
    }
  }
  std::vector<int32_t> blk;
  std::vector<TreeChunk> chunks;
  int32_t steps = 0;
  for (const Piece& pc : order) {
    const Segment& sg = segs[pc.seg];
    TreeChunk c{};
    c.blk_off = (int32_t)blk.size();
    c.n_tok = pc.n_tok;
    c.t0 = pc.t0;
    c.n_steps = (pc.n_tok + 31) / 32;
    for (int32_t b = pc.b0; b < pc.b1; ++b) blk.push_back(sg.blocks[b]);
    const int32_t need = (32 * c.n_steps + bs - 1) / bs;  // blocks the steps touch
    while ((int32_t)blk.size() - c.blk_off < need) blk.push_back(sg.blocks[pc.b1 - 1]);
    for (int32_t h = 0; h < sg.n_hold; ++h) {
      const int32_t br = S->holders[sg.hold_off + h];
      for (int32_t g = 0; g < G; ++g) {
        const int32_t r = br * G + g;
        c.rows[r >> 6] |= 1ull << (r & 63);
      }
    }
    steps += c.n_steps;
    chunks.push_back(c);
  }
  if ((int64_t)blk.size() > kMaxTreeBlocks) return false;
  TreeItem it{};
  it.hold_off = (int32_t)S->holders.size();
  it.n_rows = rows;
  it.chunk_off = 0;
  it.n_chunks = (int32_t)chunks.size();
  it.blk_off = 0;
  it.n_blk = (int32_t)blk.size();
  it.n_steps = steps;
  for (int32_t i = 0; i < n; ++i) S->holders.push_back(i);
  S->blk = std::move(blk);
  S->tchunks = std::move(chunks);
  S->titems.assign(1, it);
  S->tree = true;
  return true;
}

// Groups of sibling branches, after folding: a branch whose folded run is
// its only single-holder segment is a candidate; candidates are sorted by
// their paths of segments before folding (`key`: segment numbers, given in
// the order the batch meets them, so the groups do not depend on where the
// blocks sit in the pool), so that branches sharing a path prefix (siblings
// of a tree) sit next to each other, and cut into groups of `per`. A group
// whose union of blocks is at most 3/4 of its members' blocks becomes one
// segment: its holders (ascending), the union in first-seen order, and per
// block the bits of the holders that read it and its valid slots. Its items
// read each shared block once for all members instead of once per member.
// A block two members see with different valid counts (a kept, partly
// filled block after a truncate) enters the union once per count.
void group_runs(std::vector<Segment>& segs, std::vector<std::vector<int32_t>>& path,
                const std::vector<std::vector<int32_t>>& key, const std::vector<const Seq*>& sv,
                int32_t bs, int32_t per, Schedule* S) {
  const int32_t n = (int32_t)path.size();
  std::vector<int32_t> run(n, -1), cand;
  for (int32_t i = 0; i < n; ++i) {
    int32_t runs = 0;
    for (int32_t sgi : path[i])
      if (segs[sgi].n_hold == 1) {
        ++runs;
        run[i] = sgi;
      }
    if (runs == 1) cand.push_back(i);
  }
  std::stable_sort(cand.begin(), cand.end(), [&](int32_t a, int32_t b) {
    return std::lexicographical_compare(key[a].begin(), key[a].end(), key[b].begin(), key[b].end());
  });
  std::vector<int32_t> group_of(n, -1);
  std::vector<char> dead(segs.size(), 0);
  std::vector<Segment> groups;
  std::unordered_map<int64_t, int32_t> seen;
  for (size_t c0 = 0; c0 + 1 < cand.size(); c0 += per) {
    const size_t c1 = std::min(cand.size(), c0 + per);
    std::vector<int32_t> hs(cand.begin() + c0, cand.begin() + c1);
    std::sort(hs.begin(), hs.end());
    Segment g;
    g.t0 = 0x7fffffff;
    seen.clear();
    int64_t total = 0;
    for (size_t c = c0; c < c1; ++c) {
      const int32_t i = cand[c];
      const Segment& r = segs[run[i]];
      const int32_t bit = 1 << (int32_t)(std::lower_bound(hs.begin(), hs.end(), i) - hs.begin());
      const int32_t p0 = r.t0 / bs;
      g.t0 = std::min(g.t0, r.t0);
      for (size_t j = 0; j < r.blocks.size(); ++j) {
        const int32_t v = std::min<int32_t>(bs, sv[i]->len - (p0 + (int32_t)j) * bs);
        const int64_t key = (int64_t)r.blocks[j] * 128 + v;  // v <= 64
        auto ins = seen.emplace(key, (int32_t)g.blocks.size());
        if (ins.second) {
          g.blocks.push_back(r.blocks[j]);
          g.binfo.push_back(v << 16);
        }
        g.binfo[ins.first->second] |= bit;
      }
      total += (int64_t)r.blocks.size();
    }
    if (4 * (int64_t)g.blocks.size() > 3 * total) continue;  // too little shared
    g.n_tok = (int32_t)g.blocks.size() * bs;
    g.hold_off = (int32_t)S->holders.size();
    g.n_hold = (int32_t)hs.size();
    g.all_bits = (1 << g.n_hold) - 1;
    S->holders.insert(S->holders.end(), hs.begin(), hs.end());
    for (int32_t i : hs) {
      dead[run[i]] = 1;
      group_of[i] = (int32_t)groups.size();
    }
    groups.push_back(std::move(g));
  }
  if (groups.empty()) return;
  std::vector<Segment> out;
  std::vector<int32_t> remap(segs.size(), -1);
  for (size_t k = 0; k < segs.size(); ++k) {
    if (dead[k]) continue;
    remap[k] = (int32_t)out.size();
    out.push_back(std::move(segs[k]));
  }
  const int32_t g0 = (int32_t)out.size();
  for (Segment& g : groups) out.push_back(std::move(g));
  for (int32_t i = 0; i < n; ++i)
    for (int32_t& sgi : path[i]) sgi = dead[sgi] ? g0 + group_of[i] : remap[sgi];
  segs = std::move(out);
  S->grouped = true;
}

}  // namespace

void Schedule::build_order(int32_t n_layers, int32_t Hkv) {
  const int32_t LH = n_layers * Hkv;
  order.clear();
  // narrow launch: no table (code = blockIdx for long items; four short
  // codes per workgroup: four planes of one item, or, when short shared
  // segments were folded into per-branch items, four items of one plane with
  // a plane's workgroups 8 apart: ceil(LH / 8) groups of 8 planes,
  // ceil(n_short / 4) rounds each)
  const int64_t long_codes = (int64_t)(n_narrow - n_short) * LH;
  const int64_t short_codes = (int64_t)n_short * LH;
  const int64_t short_wgs = n_short == 0 ? 0
                            : folded  ? (int64_t)((LH + 7) / 8) * 8 * ((n_short + 3) / 4)
                                      : (short_codes + 3) / 4;
  const int64_t long_wgs = long_by_plane ? (int64_t)((LH + 7) / 8) * 8 * (n_narrow - n_short)
                                         : long_codes;
  n_long_wgs = (int32_t)long_wgs;
  n_order_narrow = (int32_t)(long_wgs + short_wgs);
  // wide launch: a unit is (sibling group, plane); the R siblings of a unit
  // are placed 8 workgroups apart, so that with workgroups dealt round-robin
  // to the 8 XCDs they share one XCD (and its L2) and start together
  struct Unit {
    int32_t first, R, lh;
  };
  std::vector<Unit> units;
  for (int32_t i = n_narrow; i < (int32_t)items.size();) {
    int32_t R = 1;
    while (i + R < (int32_t)items.size() && items[i + R].blk_off == items[i].blk_off &&
           items[i + R].r0 > items[i].r0)
      ++R;
    for (int32_t lh = 0; lh < LH; ++lh) units.push_back({i, R, lh});
    i += R;
  }
  for (size_t u = 0; u < units.size();) {
    const int32_t R = units[u].R;
    size_t k = 0;
    while (k < 8 && u + k < units.size() && units[u + k].R == R) ++k;
    for (int32_t r = 0; r < R; ++r)
      for (size_t j = 0; j < 8; ++j)
        order.push_back(j < k ? (units[u + j].first + r) * LH + units[u + j].lh : -1);
    u += k;
  }
  n_order_wide = (int32_t)order.size();
}

void Schedule::layout(int Hkv, int D) {
  // the schedule's arrays 16-byte aligned and packed (small schedules travel
  // in the launch's arguments), the partial states 256-byte aligned after them
  auto align16 = [](size_t x) { return (x + 15) & ~size_t(15); };
  size_t o = 0;
  off_items = o;
  o = align16(o + items.size() * sizeof(WorkItem));
  off_blk = o;
  o = align16(o + blk.size() * sizeof(int32_t));
  off_holders = o;
  o = align16(o + holders.size() * sizeof(int32_t));
  off_comb_ptr = o;
  o = align16(o + comb_ptr.size() * sizeof(int32_t));
  off_comb_rows = o;
  o = align16(o + comb_rows.size() * sizeof(int32_t));
  off_anc = o;
  o = align16(o + anc.size() * sizeof(uint64_t));
  off_order = o;
  o = align16(o + order.size() * sizeof(int32_t));
  off_titems = o;
  o = align16(o + titems.size() * sizeof(TreeItem));
  off_tchunks = o;
  o = align16(o + tchunks.size() * sizeof(TreeChunk));
  off_binfo = o;
  o = align16(o + binfo.size() * sizeof(int32_t));
  meta_bytes = o;
  const size_t planes = (size_t)n_layers * Hkv;
  off_ml = align256(o);
  o = align256(off_ml + planes * P * 2 * sizeof(float));
  off_acc = o;
  o = align256(o + planes * P * (size_t)D * sizeof(float));
  total_bytes = o;
}

void Schedule::pack_meta(uint8_t* dst) const {
  std::memset(dst, 0, meta_bytes);
  std::memcpy(dst + off_items, items.data(), items.size() * sizeof(WorkItem));
  std::memcpy(dst + off_blk, blk.data(), blk.size() * sizeof(int32_t));
  std::memcpy(dst + off_holders, holders.data(), holders.size() * sizeof(int32_t));
  std::memcpy(dst + off_comb_ptr, comb_ptr.data(), comb_ptr.size() * sizeof(int32_t));
  std::memcpy(dst + off_comb_rows, comb_rows.data(), comb_rows.size() * sizeof(int32_t));
  if (!anc.empty()) std::memcpy(dst + off_anc, anc.data(), anc.size() * sizeof(uint64_t));
  if (!order.empty()) std::memcpy(dst + off_order, order.data(), order.size() * sizeof(int32_t));
  if (!titems.empty()) std::memcpy(dst + off_titems, titems.data(), titems.size() * sizeof(TreeItem));
  if (!tchunks.empty())
    std::memcpy(dst + off_tchunks, tchunks.data(), tchunks.size() * sizeof(TreeChunk));
  if (!binfo.empty()) std::memcpy(dst + off_binfo, binfo.data(), binfo.size() * sizeof(int32_t));
}

void PlannerScratch::ensure(int nb) {
  if ((int)stamp.size() < nb) {
    stamp.assign(nb, 0);
    cnt.assign(nb, 0);
    pos.assign(nb, 0);
    valid.assign(nb, 0);
    off.assign(nb, 0);
    fill.assign(nb, 0);
    seg.assign(nb, -1);
    epoch = 0;
  }
  if (++epoch == 0) {  // wrapped: clear stamps
    std::fill(stamp.begin(), stamp.end(), 0);
    epoch = 1;
  }
}

int build_decode_schedule(const Pool& pool, const pkv_seq* seqs, int32_t n, int32_t n_layers,
                          int32_t layer0, const SchedOptions& opt, PlannerScratch* X,
                          Schedule* S) {
  const pkv_pool_desc& d = pool.desc();
  const int32_t bs = d.block_size, G = d.num_q_heads / d.num_kv_heads;
  if (n <= 0 || !seqs) return fail(PKV_E_INVALID, "decode: empty batch");
  if (n_layers <= 0 || layer0 < 0 || layer0 + n_layers > d.num_layers)
    return fail(PKV_E_INVALID, "decode: layer range outside the pool");
  std::vector<const Seq*> sv(n);
  for (int32_t i = 0; i < n; ++i) {
    sv[i] = pool.get(seqs[i]);
    if (!sv[i]) return PKV_E_INVALID;
    if (sv[i]->len <= 0) return fail(PKV_E_INVALID, "decode: a sequence is empty");
  }
  *S = Schedule();
  S->n_branch = n;
  S->n_layers = n_layers;
  X->ensure(d.num_blocks);
  const uint32_t ep = X->epoch;
  // pass 1: holder counts, logical position and valid slots of every block.
  // Holders of a block hold it at the same position (a fork copies a table
  // prefix), but after a truncate they may see different valid counts in
  // it (a kept, partly filled block that a sibling has filled further); such
  // a block is marked (valid -1) and each holder reads it on its own.
  std::vector<int32_t> distinct;
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = *sv[i];
    const std::vector<int32_t>& sb = pool.blocks(s);
    for (int32_t j = 0; j < (int32_t)sb.size(); ++j) {
      const int32_t b = sb[j];
      const int32_t v = std::min(bs, s.len - j * bs);
      if (X->stamp[b] != ep) {
        X->stamp[b] = ep;
        X->cnt[b] = 0;
        X->pos[b] = j;
        X->valid[b] = v;
        X->seg[b] = -1;
        distinct.push_back(b);
      } else if (X->pos[b] != j) {
        return fail(PKV_E_INVALID, "decode: a shared block sits at two logical positions");
      } else if (X->valid[b] != v) {
        X->valid[b] = -1;
      }
      ++X->cnt[b];
    }
  }
  // holder lists (ascending batch index) in one array
  std::vector<int32_t> hold_all;
  {
    int32_t o = 0;
    for (int32_t b : distinct) {
      X->off[b] = o;
      X->fill[b] = 0;
      o += X->cnt[b];
    }
    hold_all.resize(o);
    for (int32_t i = 0; i < n; ++i)
      for (int32_t b : pool.blocks(*sv[i])) hold_all[X->off[b] + X->fill[b]++] = i;
  }
  // segments: maximal runs with one holder set, found by the first holder;
  // a block read per holder (valid -1) has the holder set {i} for holder i.
  // Each branch's segments are listed in logical order as they are found.
  std::vector<Segment> segs;
  std::vector<std::vector<int32_t>> path((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = *sv[i];
    const std::vector<int32_t>& sb = pool.blocks(s);
    int32_t cur = -1;
    for (int32_t j = 0; j < (int32_t)sb.size(); ++j) {
      const int32_t b = sb[j];
      const bool own = X->valid[b] < 0;
      int32_t sgi;
      if (!own && X->seg[b] >= 0) {
        cur = -1;
        sgi = X->seg[b];
      } else {
        const int32_t* key = own ? &i : hold_all.data() + X->off[b];
        const int32_t nkey = own ? 1 : X->cnt[b];
        const int32_t v = own ? std::min(bs, s.len - j * bs) : X->valid[b];
        if (cur >= 0 && segs[cur].n_hold == nkey &&
            std::equal(key, key + nkey, S->holders.begin() + segs[cur].hold_off)) {
          segs[cur].blocks.push_back(b);
          segs[cur].n_tok += v;
        } else {
          Segment sg;
          sg.blocks.push_back(b);
          sg.t0 = j * bs;
          sg.n_tok = v;
          sg.hold_off = (int32_t)S->holders.size();
          sg.n_hold = nkey;
          S->holders.insert(S->holders.end(), key, key + nkey);
          segs.push_back(std::move(sg));
          cur = (int32_t)segs.size() - 1;
        }
        if (!own) X->seg[b] = cur;
        sgi = cur;
      }
      if (path[i].empty() || path[i].back() != sgi) path[i].push_back(sgi);
    }
  }
  S->n_segments = (int32_t)segs.size();
  for (const Segment& sg : segs) S->unique_tokens += sg.n_tok;
  // The tree launch: when all rows fit one workgroup, one workgroup per
  // plane reads every segment once (no partial states, no combine); chosen
  // automatically when some segment is wide and the planes alone fill the
  // chip (else the narrow / wide items' split of long segments is needed for
  // parallelism).
  if (opt.tree > 0 && opt.tree_ok) {
    bool wide_seg = false;
    for (const Segment& sg : segs) wide_seg = wide_seg || sg.n_hold * G > opt.rows_per_item;
    const int64_t planes = (int64_t)n_layers * d.num_kv_heads;
    const bool pays = opt.tree == 2 || (wide_seg && 4 * planes >= 3 * (int64_t)opt.target_workgroups);
    if (pays && plan_tree(segs, n, bs, G, opt.tree_piece_tokens, S)) {
      for (const Segment& sg : segs)
        if (sg.n_hold * G > opt.rows_per_item) S->wide_tokens += sg.n_tok;
      S->n_chunks = (int32_t)S->tchunks.size();
      S->n_branch = n;
      S->layout(d.num_kv_heads, d.head_dim);
      return PKV_OK;
    }
  }
  // Short shared segments are folded into per-branch segments: a shared
  // segment writes one partial state per row it serves, and when it holds
  // few tokens (an MCTS edge: 32 tokens for up to 128 rows per KV head)
  // those states outweigh its K/V; re-reading it once per branch (mostly
  // from the caches, siblings run side by side) and merging it into one
  // state per branch with the branch's other short segments costs less.
  if (opt.fold_tokens > 0) {
    const std::vector<std::vector<int32_t>> path0 = opt.group_rows > 0 ? path : decltype(path)();
    std::vector<char> fold(segs.size(), 0);
    bool any = false;
    for (size_t k = 0; k < segs.size(); ++k) {
      fold[k] = segs[k].n_hold > 1 && segs[k].n_tok < opt.fold_tokens;
      any = any || fold[k];
    }
    S->folded = any;
    if (any) {
      // a branch's private segments join its runs too (they are per-branch
      // already): a leaf's folded edges and its own tail make one item
      for (size_t k = 0; k < segs.size(); ++k) fold[k] = fold[k] || segs[k].n_hold == 1;
      std::vector<Segment> out;
      std::vector<int32_t> holders, remap(segs.size(), -1);
      for (size_t k = 0; k < segs.size(); ++k) {
        if (fold[k]) continue;
        remap[k] = (int32_t)out.size();
        Segment sg = segs[k];
        sg.hold_off = (int32_t)holders.size();
        holders.insert(holders.end(), S->holders.begin() + segs[k].hold_off,
                       S->holders.begin() + segs[k].hold_off + segs[k].n_hold);
        out.push_back(std::move(sg));
      }
      for (int32_t i = 0; i < n; ++i) {
        std::vector<int32_t> np;
        int32_t run = -1;  // this branch's open folded segment
        for (int32_t sgi : path[i]) {
          if (!fold[sgi]) {
            run = -1;
            np.push_back(remap[sgi]);
            continue;
          }
          if (run < 0) {
            Segment sg;
            sg.t0 = segs[sgi].t0;
            sg.hold_off = (int32_t)holders.size();
            sg.n_hold = 1;
            holders.push_back(i);
            run = (int32_t)out.size();
            out.push_back(std::move(sg));
            np.push_back(run);
          }
          Segment& r = out[run];
          r.blocks.insert(r.blocks.end(), segs[sgi].blocks.begin(), segs[sgi].blocks.end());
          r.n_tok += segs[sgi].n_tok;
        }
        path[i] = std::move(np);
      }
      segs = std::move(out);
      S->holders = std::move(holders);
      const int32_t rows = std::min({opt.group_rows, 16, std::max<int32_t>(1, opt.rows_per_item)});
      if (rows / G >= 2) group_runs(segs, path, path0, sv, bs, rows / G, S);
    }
  }
  const std::vector<Chunk> chunks = emit_chunks(segs, bs, G, n_layers, d.num_kv_heads, opt, S);
  // combine lists: for each branch, its segments in logical order, each
  // segment's chunks in order; the entry is the partial row of q-head
  // offset 0 of this branch in the chunk
  S->comb_ptr.resize(n + 1);
  for (int32_t i = 0; i < n; ++i) {
    S->comb_ptr[i] = (int32_t)S->comb_rows.size();
    for (int32_t sgi : path[i]) {
      const Segment& sg = segs[sgi];
      const int32_t* h0 = S->holders.data() + sg.hold_off;
      const int32_t hidx = (int32_t)(std::lower_bound(h0, h0 + sg.n_hold, i) - h0);
      for (int32_t c = sg.chunk_begin; c < sg.chunk_end; ++c)
        S->comb_rows.push_back(chunks[c].part_base + hidx * G);
    }
  }
  S->comb_ptr[n] = (int32_t)S->comb_rows.size();
  // final outputs from the narrow launch: every branch has one narrow chunk
  // and at least one wide item exists (a chunk's items are all wide or all
  // narrow, by its row count)
  if (opt.finalize && opt.wide && S->n_narrow < (int32_t)S->items.size()) {
    const int32_t rpi = std::max<int32_t>(1, opt.rows_per_item);
    bool ok = true;
    for (int32_t i = 0; i < n && ok; ++i) {
      int32_t narrow_chunks = 0;
      for (int32_t sgi : path[i]) {
        const Segment& sg = segs[sgi];
        if (sg.n_hold * G <= rpi) narrow_chunks += sg.chunk_end - sg.chunk_begin;
      }
      ok = narrow_chunks == 1;
    }
    S->finalize = ok;
  }
  (void)layer0;
  S->layout(d.num_kv_heads, d.head_dim);
  return PKV_OK;
}

int build_verify_schedule(const Pool& pool, const pkv_seq* reqs, int32_t n_req,
                          const int32_t* parents, int32_t n_nodes, const SchedOptions& opt,
                          Schedule* S) {
  const pkv_pool_desc& d = pool.desc();
  const int32_t bs = d.block_size, G = d.num_q_heads / d.num_kv_heads;
  if (n_req <= 0 || !reqs || !parents) return fail(PKV_E_INVALID, "verify: empty batch");
  if (n_nodes < 1 || n_nodes > 64) return fail(PKV_E_UNSUPPORTED, "verify: n_nodes must be 1..64");
  *S = Schedule();
  S->n_branch = n_req * n_nodes;
  S->n_layers = 1;
  S->anc.resize((size_t)n_req * n_nodes);
  std::vector<Segment> segs;
  std::vector<int32_t> ctx(n_req);
  for (int32_t r = 0; r < n_req; ++r) {
    const Seq* s = pool.get(reqs[r]);
    if (!s) return PKV_E_INVALID;
    if (s->len < n_nodes) return fail(PKV_E_INVALID, "verify: request shorter than its tree");
    for (int32_t q = 0; q < r; ++q)
      if (reqs[q].index == reqs[r].index) return fail(PKV_E_INVALID, "verify: request repeated");
    const int32_t* par = parents + (size_t)r * n_nodes;
    for (int32_t j = 0; j < n_nodes; ++j) {
      if (par[j] < -1 || par[j] >= j)
        return fail(PKV_E_INVALID, "verify: parents[j] must be -1 or an earlier node");
      uint64_t a = 1ull << j;
      if (par[j] >= 0) a |= S->anc[(size_t)r * n_nodes + par[j]];
      S->anc[(size_t)r * n_nodes + j] = a;
    }
    ctx[r] = s->len - n_nodes;
    Segment sg;
    sg.blocks = pool.blocks(*s);
    sg.t0 = 0;
    sg.n_tok = s->len;
    sg.hold_off = (int32_t)S->holders.size();
    sg.n_hold = n_nodes;
    for (int32_t j = 0; j < n_nodes; ++j) S->holders.push_back(r * n_nodes + j);
    segs.push_back(std::move(sg));
  }
  S->n_segments = n_req;
  for (const Segment& sg : segs) S->unique_tokens += sg.n_tok;
  for (int32_t r = 0; r < n_req; ++r) segs[r].mask_from = ctx[r];
  const std::vector<Chunk> chunks = emit_chunks(segs, bs, G, 1, d.num_kv_heads, opt, S);
  // combine: node j of request r reads every chunk of r, holder index j
  S->comb_ptr.resize(S->n_branch + 1);
  for (int32_t r = 0; r < n_req; ++r)
    for (int32_t j = 0; j < n_nodes; ++j) {
      const int32_t b = r * n_nodes + j;
      S->comb_ptr[b] = (int32_t)S->comb_rows.size();
      for (int32_t c = segs[r].chunk_begin; c < segs[r].chunk_end; ++c)
        S->comb_rows.push_back(chunks[c].part_base + j * G);
    }
  S->comb_ptr[S->n_branch] = (int32_t)S->comb_rows.size();
  S->layout(d.num_kv_heads, d.head_dim);
  return PKV_OK;
}

}  // namespace pkv
