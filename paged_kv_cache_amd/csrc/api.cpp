// C ABI of libpkv (declared in include/pkv.h): argument checks, the host
// pool, host-to-device staging and kernel launches. No exception leaves
// this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "pkv.h"
#include "pool.hpp"
#include "schedule.hpp"

using namespace pkv;

static_assert(kScratchBytes == (size_t)PKV_NOALLOC_WORKSPACE_BYTES,
              "the header states the static scratch's size");

namespace {

constexpr int kRing = 8;

// A slot of the pinned staging ring: the host writes the next upload only
// after the copy that last read this slot has finished.
struct Staging {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

int hip_fail(hipError_t e, const char* what) {
  return fail(PKV_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

// Event pairs bracketing kernel launches, per kernel kind.
struct KernelTimer {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> used, spare;
  ~KernelTimer() {
    for (auto& v : {&used, &spare})
      for (auto& pr : *v) {
        (void)hipEventDestroy(pr.first);
        (void)hipEventDestroy(pr.second);
      }
  }
  int take(LaunchEvents* ev) {
    std::pair<hipEvent_t, hipEvent_t> pr;
    if (!spare.empty()) {
      pr = spare.back();
      spare.pop_back();
    } else {
      hipError_t e;
      if ((e = hipEventCreate(&pr.first)) != hipSuccess) return hip_fail(e, "hipEventCreate");
      if ((e = hipEventCreate(&pr.second)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
    used.push_back(pr);
    ev->start = pr.first;
    ev->stop = pr.second;
    return PKV_OK;
  }
  int read(double* ms, int64_t* n) {
    double tot = 0;
    for (auto& pr : used) {
      hipError_t e = hipEventSynchronize(pr.second);
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
      float t = 0;
      if ((e = hipEventElapsedTime(&t, pr.first, pr.second)) != hipSuccess)
        return hip_fail(e, "hipEventElapsedTime");
      tot += t;
    }
    *ms = tot;
    *n = (int64_t)used.size();
    spare.insert(spare.end(), used.begin(), used.end());
    used.clear();
    return PKV_OK;
  }
};

enum {
  T_ATTN = 0,
  T_COMBINE = 1,
  T_APPEND = 2,
  T_WIDE = 3,
  T_SPAN = 4,
  T_GATHER = 5,
  T_TREE = 6,
  T_KINDS = 7
};

struct pkv_pool {
  explicit pkv_pool(const pkv_pool_desc& d) : pool(d) {}
  bool timing = false;
  KernelTimer timers[T_KINDS];

  // Calls launch(LaunchEvents) (returning hipError_t); with timing on, the
  // events record the kernel's own start and end.
  template <typename F>
  int timed(int kind, F&& launch, const char* what) {
    LaunchEvents ev;
    if (timing) {
      int rc = timers[kind].take(&ev);
      if (rc) return rc;
    }
    hipError_t e = launch(ev);
    if (e != hipSuccess) return hip_fail(e, what);
    return PKV_OK;
  }

  Pool pool;
  Staging ring[kRing];
  int ring_next = 0;
  void* dmeta = nullptr;  // device copy of per-call metadata (slots, copy ops)
  size_t dmeta_cap = 0;
  std::vector<uint8_t> meta_host;  // a packed plan on its way to the static scratch
  PlannerScratch scratch;
  SchedOptions opt;
  int path = 0;  // 0 auto, 1 VALU, 2 matrix cores
  int wide_waves = 0;  // compute waves per wide workgroup (4, 6, 8; 0 automatic)
  int wide_row_blocks = 0;  // 16-row blocks per wave of the wide kernel (1, 2; 0 automatic)
  int prefetch = 0;    // narrow matrix-core kernel loads one step ahead
  int concurrent = 0;  // narrow and wide launches on two streams
  int inline_plan = 1;  // small schedules travel in the launch arguments (no upload)
  int tree_stages = 5;  // LDS ring depth of the tree kernel (4 to 6)
  // wide items on the kernel with specialised waves (head_dim 64 / 128, the
  // automatic wide shape): 1 when every wide item fills more than 3/4 of its
  // 256 rows, 2 whenever the shape allows
  int wide_spec = 0;

  // A second stream (default priority) for the wide launch, so that it runs
  // beside the narrow one; created on first use, on the device current then.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  int side_stream(hipStream_t* out) {
    if (!side) {
      hipError_t e;
      if ((e = hipStreamCreateWithFlags(&side, hipStreamNonBlocking)) != hipSuccess)
        return hip_fail(e, "hipStreamCreateWithFlags");
      if ((e = hipEventCreateWithFlags(&ev_fork, hipEventDisableTiming)) != hipSuccess)
        return hip_fail(e, "hipEventCreateWithFlags");
      if ((e = hipEventCreateWithFlags(&ev_join, hipEventDisableTiming)) != hipSuccess)
        return hip_fail(e, "hipEventCreateWithFlags");
    }
    *out = side;
    return PKV_OK;
  }

  // schedule cache
  bool cache_valid = false;
  int cache_kind = -1;  // 0 decode, 1 verify
  uint64_t cache_mut = 0;
  int32_t cache_layers = 0, cache_layer0 = 0, cache_nodes = 0;
  bool cache_mfma = false;
  std::vector<pkv_seq> cache_seqs;
  std::vector<int32_t> cache_parents;
  Schedule sched;

  ~pkv_pool() {
    if (side) {
      (void)hipStreamSynchronize(side);
      (void)hipStreamDestroy(side);
    }
    if (ev_fork) (void)hipEventDestroy(ev_fork);
    if (ev_join) (void)hipEventDestroy(ev_join);
    for (Staging& s : ring) {
      if (s.ev) {
        if (s.pending) (void)hipEventSynchronize(s.ev);
        (void)hipEventDestroy(s.ev);
      }
      if (s.host) (void)hipHostFree(s.host);
    }
    if (dmeta) (void)hipFree(dmeta);
  }

  // Copies `bytes` from the pinned slot filled by `fill` to device `dst`.
  template <typename F>
  int upload(void* dst, size_t bytes, hipStream_t stream, F&& fill) {
    if (bytes == 0) return PKV_OK;
    Staging& s = ring[ring_next];
    ring_next = (ring_next + 1) % kRing;
    hipError_t e;
    if (!s.ev) {
      if ((e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming)) != hipSuccess)
        return hip_fail(e, "hipEventCreate");
    }
    if (s.pending) {
      if ((e = hipEventSynchronize(s.ev)) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
      s.pending = false;
    }
    if (s.cap < bytes) {
      if (s.host) (void)hipHostFree(s.host);
      s.host = nullptr;
      s.cap = 0;
      size_t want = bytes < 65536 ? 65536 : bytes + bytes / 2;
      if ((e = hipHostMalloc(&s.host, want, hipHostMallocDefault)) != hipSuccess)
        return hip_fail(e, "hipHostMalloc");
      s.cap = want;
    }
    fill((uint8_t*)s.host);
    if ((e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream)) != hipSuccess)
      return hip_fail(e, "hipMemcpyAsync");
    if ((e = hipEventRecord(s.ev, stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    s.pending = true;
    return PKV_OK;
  }

  int ensure_dmeta(size_t bytes, hipStream_t stream) {
    if (dmeta_cap >= bytes) return PKV_OK;
    hipError_t e;
    if (dmeta) {
      // earlier kernels on the stream may still read the old buffer
      if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      (void)hipFree(dmeta);
      dmeta = nullptr;
      dmeta_cap = 0;
    }
    size_t want = bytes < 65536 ? 65536 : bytes + bytes / 2;
    if ((e = hipMalloc(&dmeta, want)) != hipSuccess) return hip_fail(e, "hipMalloc");
    dmeta_cap = want;
    return PKV_OK;
  }
};

namespace {

bool pool_ok(const pkv_pool* p) { return p != nullptr; }

int check_desc(const pkv_pool_desc* d) {
  if (!d) return fail(PKV_E_INVALID, "null desc");
  if (d->num_blocks <= 0 || d->block_size <= 0 || d->num_layers <= 0 || d->num_kv_heads <= 0 ||
      d->num_q_heads <= 0 || d->head_dim <= 0)
    return fail(PKV_E_INVALID, "pool sizes must be positive");
  if (d->num_q_heads % d->num_kv_heads)
    return fail(PKV_E_INVALID, "num_q_heads must be a multiple of num_kv_heads");
  if (d->kv_dtype != PKV_F32 && d->kv_dtype != PKV_BF16) return fail(PKV_E_INVALID, "bad kv_dtype");
  if ((int64_t)d->num_blocks * d->block_size > (int64_t)INT32_MAX)
    return fail(PKV_E_INVALID, "num_blocks * block_size overflows a slot id");
  const size_t es = d->kv_dtype == PKV_F32 ? 4 : 2;
  if ((d->head_dim * es) % 16)
    return fail(PKV_E_INVALID, "head_dim * element size must be a multiple of 16 bytes");
  if (d->alloc_order) {
    std::vector<char> seen(d->num_blocks, 0);
    for (int32_t i = 0; i < d->num_blocks; ++i) {
      int32_t b = d->alloc_order[i];
      if (b < 0 || b >= d->num_blocks || seen[b])
        return fail(PKV_E_INVALID, "alloc_order is not a permutation of the block ids");
      seen[b] = 1;
    }
  }
  return PKV_OK;
}

size_t elem_size(const pkv_pool_desc& d) { return d.kv_dtype == PKV_F32 ? 4 : 2; }

bool has_arenas(const pkv_pool_desc& d) { return d.k_arena && d.v_arena; }

// Copy-on-write copies and token writes of one append, in one launch. The
// tokens that land in a copy's destination block go with the copy (the
// copy workgroup assembles that block); the rest form the write list.
// Short lists travel in the kernel arguments; longer ones are staged to the
// pool's device metadata buffer in one upload.
int enqueue_append(pkv_pool* p, const pkv_cow_op* ops, int32_t n_ops, const int64_t* slots,
                   int32_t n_tok, const void* k_new, const void* v_new, hipStream_t stream) {
  if (n_ops == 0 && n_tok == 0) return PKV_OK;
  const pkv_pool_desc& d = p->pool.desc();
  if (!append_supported(d.block_size))
    return fail(PKV_E_UNSUPPORTED, "device append: block_size must be 16, 32 or 64");
  const int64_t bs = d.block_size;
  // per op: src, dst, n_valid, tok0, m
  std::vector<int32_t> op5((size_t)n_ops * 5);
  for (int32_t o = 0; o < n_ops; ++o) {
    op5[5 * o] = ops[o].src;
    op5[5 * o + 1] = ops[o].dst;
    op5[5 * o + 2] = ops[o].n_valid;
    op5[5 * o + 3] = 0;
    op5[5 * o + 4] = 0;
  }
  std::vector<int64_t> wslot;
  std::vector<int32_t> wtok;
  wslot.reserve(n_tok);
  wtok.reserve(n_tok);
  for (int32_t t = 0; t < n_tok; ++t) {
    const int64_t b = slots[t] / bs;
    int32_t hit = -1;
    for (int32_t o = 0; o < n_ops; ++o)
      if (ops[o].dst == b) {
        hit = o;
        break;
      }
    if (hit >= 0) {
      int32_t* q = &op5[5 * hit];
      if (q[4] == 0) q[3] = t;
      if (t != q[3] + q[4] || slots[t] != b * bs + q[2] + q[4])
        return fail(PKV_E_INVALID, "append: tokens in a copied block must follow its valid slots");
      ++q[4];
    } else {
      wslot.push_back(slots[t]);
      wtok.push_back(t);
    }
  }
  // A write normally never touches a copy's source (the source is shared, so
  // nobody writes it in place). After a truncate it can: two holders may see
  // different valid counts in one block, and once the longer holder's copy
  // is planned the shorter one holds the block alone and writes in place at
  // an offset the copy still reads. Then the copies run in a launch of
  // their own, before the writes, on the same stream.
  bool ordered = false;
  for (int32_t o = 0; o < n_ops && !ordered; ++o)
    for (size_t i = 0; i < wslot.size(); ++i)
      if (wslot[i] / bs == ops[o].src && wslot[i] % bs < ops[o].n_valid) {
        ordered = true;
        break;
      }
  AppendParams a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_arena = d.k_arena;
  a.v_arena = d.v_arena;
  a.n_ops = n_ops;
  a.n_write = (int32_t)wslot.size();
  a.n_tok = n_tok;
  a.L = d.num_layers;
  a.NB = d.num_blocks;
  a.Hkv = d.num_kv_heads;
  a.D = d.head_dim;
  a.BS = d.block_size;
  if (n_ops <= kInlineOps && a.n_write <= kInlineSlots) {
    std::memcpy(a.inl_ops, op5.data(), op5.size() * sizeof(int32_t));
    for (int32_t i = 0; i < a.n_write; ++i) {
      a.inl_slots[i] = wslot[i];
      a.inl_tok[i] = wtok[i];
    }
  } else {
    const size_t b_slots = (size_t)a.n_write * sizeof(int64_t);
    const size_t o_tok = (b_slots + 255) & ~size_t(255);
    const size_t b_tok = (size_t)a.n_write * sizeof(int32_t);
    const size_t o_ops = (o_tok + b_tok + 255) & ~size_t(255);
    const size_t bytes = o_ops + op5.size() * sizeof(int32_t);
    int rc = p->ensure_dmeta(bytes, stream);
    if (rc) return rc;
    rc = p->upload(p->dmeta, bytes, stream, [&](uint8_t* h) {
      if (b_slots) std::memcpy(h, wslot.data(), b_slots);
      if (b_tok) std::memcpy(h + o_tok, wtok.data(), b_tok);
      if (!op5.empty()) std::memcpy(h + o_ops, op5.data(), op5.size() * sizeof(int32_t));
    });
    if (rc) return rc;
    uint8_t* base = (uint8_t*)p->dmeta;
    a.wslots = (const int64_t*)base;
    a.wtok = (const int32_t*)(base + o_tok);
    a.ops = (const int32_t*)(base + o_ops);
  }
  if (ordered) {
    AppendParams copies = a;
    copies.n_write = 0;
    int rc = p->timed(
        T_APPEND,
        [&](const LaunchEvents& ev) { return launch_append(d.kv_dtype, copies, stream, ev); },
        "append launch");
    if (rc) return rc;
    a.n_ops = 0;
  }
  return p->timed(
      T_APPEND, [&](const LaunchEvents& ev) { return launch_append(d.kv_dtype, a, stream, ev); },
      "append launch");
}

bool use_mfma(const pkv_pool* p) {
  const pkv_pool_desc& d = p->pool.desc();
  if (p->path == 1) return false;
  return attn_supported(true, d.kv_dtype, d.head_dim, d.block_size);
}

// The planner options for the kernel path in use.
SchedOptions planner_options(const pkv_pool* p, bool mfma) {
  SchedOptions o = p->opt;
  const bool wide_head = p->pool.desc().head_dim > 128;
  if (o.min_chunk_tokens == 0) o.min_chunk_tokens = wide_head ? 768 : 1024;
  if (o.tokens_per_row == 0) o.tokens_per_row = wide_head ? 32 : 64;
  if (!mfma) {
    o.rows_per_item = std::min<int32_t>(o.rows_per_item, 16);
    o.wide = false;
    o.max_row_blocks_per_wave = 1;
    o.short_items = false;
    o.group_rows = 0;  // (the vector kernel has no per-block row masks)
  } else {
    o.tree_ok = p->pool.desc().kv_dtype == PKV_BF16 &&
                tree_supported(p->pool.desc().head_dim, p->pool.desc().block_size);
    if (attn_max_row_blocks_per_wave(p->pool.desc().head_dim) < 2 || p->prefetch)
      o.max_row_blocks_per_wave = 1;
    // a wide item holds at most what one workgroup of the wide kernel serves
    int w = p->wide_waves, r = p->wide_row_blocks;
    attn_wide_shape(p->pool.desc().head_dim, &w, &r);
    o.wide_rows = std::min<int32_t>(o.wide_rows, 16 * w * r);
  }
  return o;
}

// Builds (or reuses) the decode schedule for these arguments.
int decode_schedule(pkv_pool* p, const pkv_seq* seqs, int32_t n, int32_t layer0, int32_t n_layers) {
  // (checked before the cache comparison reads the caller's array)
  if (n <= 0 || !seqs) return fail(PKV_E_INVALID, "decode: empty batch or null sequence array");
  const bool mfma = use_mfma(p);
  if (p->cache_valid && p->cache_kind == 0 && p->cache_mut == p->pool.mutation() &&
      p->cache_layers == n_layers && p->cache_layer0 == layer0 && p->cache_mfma == mfma &&
      (int32_t)p->cache_seqs.size() == n &&
      std::memcmp(p->cache_seqs.data(), seqs, sizeof(pkv_seq) * n) == 0)
    return PKV_OK;
  p->cache_valid = false;
  const SchedOptions o = planner_options(p, mfma);
  int rc = build_decode_schedule(p->pool, seqs, n, n_layers, layer0, o, &p->scratch, &p->sched);
  if (rc) return rc;
  p->cache_valid = true;
  p->cache_kind = 0;
  p->cache_mut = p->pool.mutation();
  p->cache_layers = n_layers;
  p->cache_layer0 = layer0;
  p->cache_mfma = mfma;
  p->cache_seqs.assign(seqs, seqs + n);
  return PKV_OK;
}

int verify_schedule(pkv_pool* p, const pkv_seq* reqs, int32_t n_req, const int32_t* parents,
                    int32_t n_nodes) {
  // (checked before the cache comparison reads the caller's arrays)
  if (n_req <= 0 || !reqs || !parents)
    return fail(PKV_E_INVALID, "verify: empty batch or null request or parent array");
  const size_t np = (size_t)n_req * (size_t)(n_nodes > 0 ? n_nodes : 0);
  if (p->cache_valid && p->cache_kind == 1 && p->cache_mut == p->pool.mutation() &&
      p->cache_nodes == n_nodes && (int32_t)p->cache_seqs.size() == n_req &&
      std::memcmp(p->cache_seqs.data(), reqs, sizeof(pkv_seq) * n_req) == 0 &&
      p->cache_parents.size() == np &&
      std::memcmp(p->cache_parents.data(), parents, np * sizeof(int32_t)) == 0)
    return PKV_OK;
  p->cache_valid = false;
  int rc = build_verify_schedule(p->pool, reqs, n_req, parents, n_nodes, planner_options(p, true),
                                 &p->sched);
  if (rc) return rc;
  p->cache_valid = true;
  p->cache_kind = 1;
  p->cache_mut = p->pool.mutation();
  p->cache_nodes = n_nodes;
  p->cache_seqs.assign(reqs, reqs + n_req);
  p->cache_parents.assign(parents, parents + np);
  return PKV_OK;
}

// Uploads the schedule into the workspace and launches attention + combine.
// no_alloc (pkv_decode_attn_noalloc): ws is the static scratch array; a
// schedule too large for the launch arguments is written into it through
// copy-kernel arguments (no pinned staging), the wide launch stays on the
// caller's stream and no timing events are created or recorded.
int run_attention(pkv_pool* p, bool mfma, int32_t layer0, const void* q, float* out, float scale,
                  void* ws, size_t ws_bytes, hipStream_t stream, bool no_alloc = false) {
  const pkv_pool_desc& d = p->pool.desc();
  const Schedule& S = p->sched;
  if (!ws || ws_bytes < S.total_bytes)
    return fail(PKV_E_WORKSPACE, "workspace too small: need " + std::to_string(S.total_bytes) +
                                     " bytes, got " + std::to_string(ws_bytes));
  if ((uintptr_t)ws % 256) return fail(PKV_E_INVALID, "workspace must be 256-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_E_INVALID, "scale must be finite");
  uint8_t* w = (uint8_t*)ws;
  // A schedule that fits in the launch arguments (the combine's lists in
  // its own) goes with the launches; otherwise it is staged and copied into
  // the workspace first.
  const size_t list_bytes = S.off_anc - S.off_comb_ptr;  // comb_ptr, comb_rows
  const bool inl = p->inline_plan && S.meta_bytes <= (size_t)kInlineMetaBytes &&
                   list_bytes <= (size_t)kInlineListBytes;
  int rc = PKV_OK;
  AttnParams a;
  if (inl) {
    S.pack_meta(a.meta.b);
  } else if (no_alloc) {
    p->meta_host.resize(S.meta_bytes);
    S.pack_meta(p->meta_host.data());
    hipError_t e = launch_arg_copy(w, p->meta_host.data(), S.meta_bytes, stream);
    if (e != hipSuccess) return hip_fail(e, "plan copy launch");
  } else {
    rc = p->upload(w, S.meta_bytes, stream, [&](uint8_t* h) { S.pack_meta(h); });
    if (rc) return rc;
  }
  a.k_arena = d.k_arena;
  a.v_arena = d.v_arena;
  a.q = q;
  a.part_ml = (float*)(w + S.off_ml);
  a.part_acc = (float*)(w + S.off_acc);
  a.meta_dev = w;
  a.meta_inline = inl ? 1 : 0;
  a.off_items = (int32_t)S.off_items;
  a.off_blk = (int32_t)S.off_blk;
  a.off_holders = (int32_t)S.off_holders;
  a.off_anc = (int32_t)S.off_anc;
  a.off_order = (int32_t)S.off_order;
  a.off_comb_ptr = (int32_t)S.off_comb_ptr;
  a.off_comb_rows = (int32_t)S.off_comb_rows;
  a.off_titems = (int32_t)S.off_titems;
  a.off_tchunks = (int32_t)S.off_tchunks;
  a.off_binfo = (int32_t)S.off_binfo;
  a.n_order = S.n_order_narrow;
  a.n_long = (S.n_narrow - S.n_short) * S.n_layers * d.num_kv_heads;
  a.n_long_wgs = S.n_long_wgs;
  a.long_by_plane = S.long_by_plane ? 1 : 0;
  a.n_codes = S.n_narrow * S.n_layers * d.num_kv_heads;
  a.short_by_plane = S.folded ? 1 : 0;
  a.out = out;
  a.finalize = 0;  // set below, once the launches' streams are known
  a.n_items = (int32_t)S.items.size();
  a.n_layers = S.n_layers;
  a.layer0 = layer0;
  a.num_blocks = d.num_blocks;
  a.Hkv = d.num_kv_heads;
  a.G = d.num_q_heads / d.num_kv_heads;
  a.Hq = d.num_q_heads;
  a.n_branch = S.n_branch;
  a.P = S.P;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.abs_scale_log2 = std::max(std::fabs(a.scale_log2), 1e-30f);
  a.q_flip = scale < 0.f ? 0x80008000u : 0u;
  // P enters P.V as bf16 plus its bf16 rounding residual: with P alone in
  // bf16 a row whose weight sits on a few keys is off by up to 2^-9 |v|
  const bool lo_split = true;
  // With both launches present the wide one runs on the side stream, forked
  // from and joined back into the caller's stream: the two read disjoint
  // chunks and write disjoint partial rows, and together they keep more
  // loads in flight than either alone.
  const bool fork = a.n_order > 0 && S.n_order_wide > 0 && p->concurrent && !no_alloc;
  // (timing events are created on first use: not in the no-allocation form)
  const bool timing = p->timing;
  if (no_alloc) p->timing = false;
  struct Restore {
    pkv_pool* p;
    bool t;
    ~Restore() { p->timing = t; }
  } restore{p, timing};
  if (S.tree) {
    // one launch: every chunk read once by each plane's workgroup, final rows
    const int n_wg = (int)S.titems.size() * S.n_layers * d.num_kv_heads;
    return p->timed(
        T_TREE,
        [&](const LaunchEvents& ev) {
          return launch_attn_tree(d.head_dim, d.block_size, p->tree_stages, a, n_wg, stream, ev);
        },
        "tree attention launch");
  }
  // the narrow launch writes the outputs itself when the plan allows it and
  // the wide launch precedes it on the same stream
  a.finalize = (S.finalize && mfma && !fork && a.n_order > 0) ? 1 : 0;
  hipStream_t wstream = stream;
  LaunchEvents span;  // both attention launches, start to end, on the caller's stream
  if (p->timing) {
    if ((rc = p->timers[T_SPAN].take(&span))) return rc;
    hipError_t e = hipEventRecord(span.start, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  if (fork) {
    if ((rc = p->side_stream(&wstream))) return rc;
    hipError_t e;
    if ((e = hipEventRecord(p->ev_fork, stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(wstream, p->ev_fork, 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
  }
  if (S.n_order_wide > 0) {
    // the specialised kernel serves 256 rows per workgroup in four pairs of
    // waves, each pair computing four 16-row blocks whether or not they hold
    // rows: taken only when every wide item is more than 3/4 full
    bool use_spec = false;
    if (p->wide_spec && d.kv_dtype == PKV_BF16 && spec_supported(d.head_dim, d.block_size)) {
      int w = p->wide_waves, r = p->wide_row_blocks;
      attn_wide_shape(d.head_dim, &w, &r);
      use_spec = 16 * w * r == spec_rows();
      for (size_t i = (size_t)S.n_narrow; use_spec && p->wide_spec == 1 && i < S.items.size(); ++i)
        use_spec = 4 * S.items[i].n_rows > 3 * spec_rows();
    }
    AttnParams aw = a;
    aw.n_order = S.n_order_wide;
    rc = p->timed(
        T_WIDE,
        [&](const LaunchEvents& ev) {
          int w = p->wide_waves, r = p->wide_row_blocks;
          attn_wide_shape(d.head_dim, &w, &r);
          if (use_spec) return launch_attn_spec(d.head_dim, d.block_size, aw, wstream, ev);
          return launch_attn_wide(d.head_dim, d.block_size, w, r, aw, wstream, ev);
        },
        "wide attention launch");
    if (rc) return rc;
  }
  if (a.n_order > 0) {
    rc = p->timed(
        T_ATTN,
        [&](const LaunchEvents& ev) {
          return launch_attn(mfma, lo_split, p->prefetch != 0, S.narrow_rw, d.kv_dtype,
                             d.head_dim, d.block_size, a, stream, ev);
        },
        "attention launch");
    if (rc) return rc;
  }
  if (fork) {
    hipError_t e;
    if ((e = hipEventRecord(p->ev_join, wstream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(stream, p->ev_join, 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
  }
  if (p->timing) {
    hipError_t e = hipEventRecord(span.stop, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  if (a.finalize) return PKV_OK;
  CombineParams c;
  c.part_ml = a.part_ml;
  c.part_acc = a.part_acc;
  c.meta_dev = w;
  c.lists_inline = inl ? 1 : 0;
  c.off_comb_ptr = (int32_t)S.off_comb_ptr;
  c.off_comb_rows = (int32_t)S.off_comb_rows;
  if (inl) {
    // the lists keep their offsets relative to the first of them
    std::memcpy(c.lists, a.meta.b + S.off_comb_ptr, list_bytes);
    c.off_comb_ptr = 0;
    c.off_comb_rows = (int32_t)(S.off_comb_rows - S.off_comb_ptr);
  }
  c.out = out;
  c.n_layers = S.n_layers;
  c.n_branch = S.n_branch;
  c.Hkv = a.Hkv;
  c.G = a.G;
  c.Hq = a.Hq;
  c.P = S.P;
  int32_t max_entries = 0;
  for (int32_t b = 0; b < S.n_branch; ++b)
    max_entries = std::max(max_entries, S.comb_ptr[b + 1] - S.comb_ptr[b]);
  return p->timed(
      T_COMBINE,
      [&](const LaunchEvents& ev) { return launch_combine(d.head_dim, max_entries, c, stream, ev); },
      "combine launch");
}

}  // namespace

#define PKV_GUARD_BEGIN \
  clear_error();        \
  try {
#define PKV_GUARD_END                                         \
  }                                                           \
  catch (const std::bad_alloc&) {                             \
    return fail(PKV_E_OOM, "host allocation failed");         \
  }                                                           \
  catch (...) {                                               \
    return fail(PKV_E_INVALID, "unexpected internal error");  \
  }

extern "C" {

int pkv_pool_create(const pkv_pool_desc* desc, pkv_pool** out) {
  PKV_GUARD_BEGIN
  if (!out) return fail(PKV_E_INVALID, "null output");
  int rc = check_desc(desc);
  if (rc) return rc;
  *out = new pkv_pool(*desc);
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_pool_destroy(pkv_pool* pool) {
  PKV_GUARD_BEGIN
  if (!pool) return fail(PKV_E_INVALID, "null pool");
  delete pool;
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_block_alloc(pkv_pool* pool, int32_t* id) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.block_alloc(id);
  PKV_GUARD_END
}

int pkv_block_release(pkv_pool* pool, int32_t id) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.block_release(id);
  PKV_GUARD_END
}

int pkv_seq_create(pkv_pool* pool, pkv_seq* out) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.seq_create(out);
  PKV_GUARD_END
}

int pkv_seq_fork(pkv_pool* pool, pkv_seq parent, pkv_seq* child) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.seq_fork(parent, child);
  PKV_GUARD_END
}

int pkv_seq_free(pkv_pool* pool, pkv_seq seq) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.seq_free(seq);
  PKV_GUARD_END
}

int pkv_seq_fork_many(pkv_pool* pool, const pkv_seq* parents, int32_t n, pkv_seq* children) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  if (n < 0 || (n > 0 && (!parents || !children))) return fail(PKV_E_INVALID, "fork_many: bad arguments");
  for (int32_t i = 0; i < n; ++i)
    if (!pool->pool.get(parents[i])) return PKV_E_INVALID;
  for (int32_t i = 0; i < n; ++i) {
    int rc = pool->pool.seq_fork(parents[i], &children[i]);
    if (rc) {  // cannot happen after the checks (host allocation aside): undo
      for (int32_t j = 0; j < i; ++j) (void)pool->pool.seq_free(children[j]);
      return rc;
    }
  }
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_seq_free_many(pkv_pool* pool, const pkv_seq* seqs, int32_t n) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  if (n < 0 || (n > 0 && !seqs)) return fail(PKV_E_INVALID, "free_many: bad arguments");
  // every handle valid and listed once (sorted slot indexes; the check is
  // all-or-nothing, before anything is freed)
  std::vector<uint32_t> idx((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    if (!pool->pool.get(seqs[i])) return PKV_E_INVALID;
    idx[i] = (uint32_t)seqs[i].index;
  }
  std::sort(idx.begin(), idx.end());
  if (std::adjacent_find(idx.begin(), idx.end()) != idx.end())
    return fail(PKV_E_INVALID, "free_many: handle listed twice");
  for (int32_t i = 0; i < n; ++i) (void)pool->pool.seq_free(seqs[i]);
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_seq_append_plan(pkv_pool* pool, pkv_seq seq, int32_t n, int64_t* slots_out,
                        pkv_cow_op* cow_out, int32_t* n_cow) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  if (n < 0) return fail(PKV_E_INVALID, "append: negative token count");
  if ((n > 0 && !slots_out) || !cow_out || !n_cow) return fail(PKV_E_INVALID, "append: null buffer");
  std::vector<int64_t> slots;
  std::vector<pkv_cow_op> cows;
  int rc = pool->pool.append_plan_batch(&seq, &n, 1, &slots, &cows);
  if (rc) return rc;
  if (n) std::memcpy(slots_out, slots.data(), sizeof(int64_t) * slots.size());
  *n_cow = (int32_t)cows.size();
  if (!cows.empty()) *cow_out = cows[0];
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_cow_copy(pkv_pool* pool, const pkv_cow_op* ops, int32_t n, void* stream) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  const pkv_pool_desc& d = pool->pool.desc();
  if (!has_arenas(d)) return fail(PKV_E_INVALID, "pool has no device arenas");
  if (n < 0 || (n > 0 && !ops)) return fail(PKV_E_INVALID, "cow_copy: bad op list");
  for (int32_t i = 0; i < n; ++i) {
    const pkv_cow_op& o = ops[i];
    if (o.src < 0 || o.src >= d.num_blocks || o.dst < 0 || o.dst >= d.num_blocks || o.n_valid < 0 ||
        o.n_valid > d.block_size)
      return fail(PKV_E_INVALID, "cow_copy: op out of range");
  }
  if ((int64_t)n * d.num_layers > INT32_MAX) return fail(PKV_E_INVALID, "cow_copy: too many ops");
  return enqueue_append(pool, ops, n, nullptr, 0, nullptr, nullptr, (hipStream_t)stream);
  PKV_GUARD_END
}

int pkv_write_kv(pkv_pool* pool, const int64_t* slots, int32_t n, const void* k_new,
                 const void* v_new, void* stream) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  const pkv_pool_desc& d = pool->pool.desc();
  if (!has_arenas(d)) return fail(PKV_E_INVALID, "pool has no device arenas");
  if (n < 0 || (n > 0 && (!slots || !k_new || !v_new))) return fail(PKV_E_INVALID, "write_kv: bad arguments");
  const int64_t max_slot = (int64_t)d.num_blocks * d.block_size;
  for (int32_t i = 0; i < n; ++i)
    if (slots[i] < 0 || slots[i] >= max_slot) return fail(PKV_E_INVALID, "write_kv: slot out of range");
  return enqueue_append(pool, nullptr, 0, slots, n, k_new, v_new, (hipStream_t)stream);
  PKV_GUARD_END
}

int pkv_append_kv_batch(pkv_pool* pool, const pkv_seq* seqs, const int32_t* counts, int32_t n_seqs,
                        const void* k_new, const void* v_new, void* stream) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  const pkv_pool_desc& d = pool->pool.desc();
  if (!has_arenas(d)) return fail(PKV_E_INVALID, "pool has no device arenas");
  int64_t total = 0;
  for (int32_t i = 0; i < n_seqs; ++i) total += counts ? counts[i] : 0;
  if (total > 0 && (!k_new || !v_new)) return fail(PKV_E_INVALID, "append: null K/V");
  if (total > INT32_MAX) return fail(PKV_E_INVALID, "append: too many tokens");
  std::vector<int64_t> slots;
  std::vector<pkv_cow_op> cows;
  slots.reserve((size_t)total);
  int rc = pool->pool.append_plan_batch(seqs, counts, n_seqs, &slots, &cows);
  if (rc) return rc;
  // The tables are updated; a device failure below leaves them updated
  // (the error is PKV_E_HIP, after which the device state is unknown).
  return enqueue_append(pool, cows.data(), (int32_t)cows.size(), slots.data(),
                        (int32_t)slots.size(), k_new, v_new, (hipStream_t)stream);
  PKV_GUARD_END
}

int pkv_seq_append_kv(pkv_pool* pool, pkv_seq seq, int32_t n, const void* k_new, const void* v_new,
                      void* stream) {
  return pkv_append_kv_batch(pool, &seq, &n, 1, k_new, v_new, stream);
}

int pkv_seq_truncate(pkv_pool* pool, pkv_seq seq, int32_t new_len) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.seq_truncate(seq, new_len);
  PKV_GUARD_END
}

int pkv_tree_commit_workspace_size(const pkv_pool* pool, int32_t n_accepted, size_t* bytes) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool) || !bytes) return fail(PKV_E_INVALID, "null argument");
  if (n_accepted < 0) return fail(PKV_E_INVALID, "commit: negative token count");
  const pkv_pool_desc& d = pool->pool.desc();
  const size_t half = ((size_t)d.num_layers * n_accepted * d.num_kv_heads * d.head_dim *
                           elem_size(d) + 255) & ~size_t(255);
  *bytes = 2 * half;
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_tree_commit_batch(pkv_pool* pool, const pkv_seq* seqs, int32_t n_req, int32_t n_nodes,
                          const int32_t* parents, const int32_t* accepted,
                          const int32_t* n_accepted, void* ws, size_t ws_bytes, void* stream) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  const pkv_pool_desc& d = pool->pool.desc();
  if (!has_arenas(d)) return fail(PKV_E_INVALID, "pool has no device arenas");
  if (!append_supported(d.block_size))
    return fail(PKV_E_UNSUPPORTED, "commit: block_size must be 16, 32 or 64");
  if (n_req < 1 || !seqs || !parents || !n_accepted)
    return fail(PKV_E_INVALID, "commit: empty batch or null argument");
  if (n_nodes < 1 || n_nodes > 64) return fail(PKV_E_INVALID, "commit: n_nodes must be 1..64");
  int64_t total = 0;
  for (int32_t r = 0; r < n_req; ++r) {
    const int32_t na = n_accepted[r];
    if (na < 0 || na > n_nodes) return fail(PKV_E_INVALID, "commit: n_accepted outside [0, n_nodes]");
    if (na > 0 && !accepted) return fail(PKV_E_INVALID, "commit: null argument");
    const int32_t* par = parents + (size_t)r * n_nodes;
    for (int32_t j = 0; j < n_nodes; ++j)
      if (par[j] < -1 || par[j] >= j) return fail(PKV_E_INVALID, "commit: bad parent pointer");
    const int32_t* acc = accepted ? accepted + (size_t)r * n_nodes : nullptr;
    int32_t prev = -1;
    for (int32_t i = 0; i < na; ++i) {
      const int32_t a = acc[i];
      if (a < 0 || a >= n_nodes || par[a] != prev)
        return fail(PKV_E_INVALID, "commit: accepted nodes are not a chain from a root");
      prev = a;
    }
    const Seq* s = pool->pool.get(seqs[r]);
    if (!s) return PKV_E_INVALID;
    if (s->len < n_nodes) return fail(PKV_E_INVALID, "commit: a sequence is shorter than its tree");
    total += na;
  }
  if (total > INT32_MAX / 2) return fail(PKV_E_INVALID, "commit: too many tokens");
  size_t need = 0;
  int rc = pkv_tree_commit_workspace_size(pool, (int32_t)total, &need);
  if (rc) return rc;
  if (total > 0 && (!ws || ws_bytes < need)) return fail(PKV_E_WORKSPACE, "commit: workspace too small");
  // slots of the kept nodes, read from the tables before they change
  const int64_t bs = d.block_size;
  std::vector<int64_t> gslots;
  std::vector<int32_t> keep((size_t)n_req);
  gslots.reserve((size_t)total);
  for (int32_t r = 0; r < n_req; ++r) {
    const Seq* s = pool->pool.get(seqs[r]);
    const std::vector<int32_t>& t = pool->pool.blocks(*s);
    keep[r] = s->len - n_nodes;
    for (int32_t i = 0; i < n_accepted[r]; ++i) {
      const int64_t pos = (int64_t)keep[r] + accepted[(size_t)r * n_nodes + i];
      gslots.push_back((int64_t)t[(size_t)(pos / bs)] * bs + pos % bs);
    }
  }
  // tables (all or nothing), then the device work: the gathers read the
  // kept nodes before the append overwrites or reuses their slots
  std::vector<int64_t> slots;
  std::vector<pkv_cow_op> cows;
  if ((rc = pool->pool.truncate_append_batch(seqs, keep.data(), n_accepted, n_req, &slots, &cows)))
    return rc;
  if (total == 0) return PKV_OK;
  hipStream_t strm = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  const size_t half = need / 2;
  for (int64_t g0 = 0; g0 < total; g0 += kGatherSlots) {
    GatherParams g{};
    g.k_arena = d.k_arena;
    g.v_arena = d.v_arena;
    g.k_out = w;
    g.v_out = w + half;
    g.n = (int32_t)std::min<int64_t>(kGatherSlots, total - g0);
    g.row0 = (int32_t)g0;
    g.n_rows = (int32_t)total;
    g.L = d.num_layers;
    g.NB = d.num_blocks;
    g.Hkv = d.num_kv_heads;
    g.D = d.head_dim;
    g.BS = d.block_size;
    for (int32_t i = 0; i < g.n; ++i) g.slots[i] = gslots[(size_t)(g0 + i)];
    rc = pool->timed(
        T_GATHER, [&](const LaunchEvents& ev) { return launch_gather(d.kv_dtype, g, strm, ev); },
        "gather launch");
    if (rc) return rc;
  }
  return enqueue_append(pool, cows.data(), (int32_t)cows.size(), slots.data(),
                        (int32_t)slots.size(), w, w + half, strm);
  PKV_GUARD_END
}

int pkv_tree_commit(pkv_pool* pool, pkv_seq seq, int32_t n_nodes, const int32_t* parents,
                    const int32_t* accepted, int32_t n_accepted, void* ws, size_t ws_bytes,
                    void* stream) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  if (n_nodes < 1 || n_nodes > 64) return fail(PKV_E_INVALID, "commit: n_nodes must be 1..64");
  if (n_accepted < 0 || n_accepted > n_nodes)
    return fail(PKV_E_INVALID, "commit: n_accepted outside [0, n_nodes]");
  if (n_accepted > 0 && !accepted) return fail(PKV_E_INVALID, "commit: null argument");
  int32_t row[64];
  for (int32_t i = 0; i < n_accepted; ++i) row[i] = accepted[i];
  return pkv_tree_commit_batch(pool, &seq, 1, n_nodes, parents, n_accepted ? row : nullptr,
                               &n_accepted, ws, ws_bytes, stream);
  PKV_GUARD_END
}

int pkv_prefix_insert(pkv_pool* pool, pkv_seq seq, const int32_t* tokens, int32_t n_tokens,
                      int32_t* n_added) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.prefix_insert(seq, tokens, n_tokens, n_added);
  PKV_GUARD_END
}

int pkv_prefix_match(pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, pkv_seq* out,
                     int32_t* n_matched) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.prefix_match(tokens, n_tokens, out, n_matched);
  PKV_GUARD_END
}

int pkv_prefix_clear(pkv_pool* pool) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  pool->pool.prefix_clear();
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_prefix_info(const pkv_pool* pool, int32_t* entries, int32_t* evictable) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  if (entries) *entries = pool->pool.prefix_entries();
  if (evictable) *evictable = pool->pool.prefix_evictable();
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_seq_info(const pkv_pool* pool, pkv_seq seq, int32_t* len, int32_t* n_blocks) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.seq_info(seq, len, n_blocks);
  PKV_GUARD_END
}

int pkv_seq_blocks(const pkv_pool* pool, pkv_seq seq, int32_t* out, int32_t cap) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.seq_blocks(seq, out, cap);
  PKV_GUARD_END
}

int pkv_block_refcount(const pkv_pool* pool, int32_t id, int32_t* count) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.refcount(id, count);
  PKV_GUARD_END
}

int pkv_block_refcounts(const pkv_pool* pool, int32_t* counts, int32_t n) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.refcounts(counts, n);
  PKV_GUARD_END
}

int pkv_pool_stats(const pkv_pool* pool, pkv_stats* stats) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  return pool->pool.stats(stats);
  PKV_GUARD_END
}

int pkv_arena_bytes(const pkv_pool_desc* desc, size_t* bytes) {
  PKV_GUARD_BEGIN
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return fail(PKV_E_INVALID, "null output");
  *bytes = (size_t)desc->num_layers * desc->num_blocks * desc->num_kv_heads * desc->block_size *
           desc->head_dim * elem_size(*desc);
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_decode_workspace_size(pkv_pool* pool, const pkv_seq* seqs, int32_t n_seqs, int32_t n_layers,
                              size_t* bytes) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool) || !bytes) return fail(PKV_E_INVALID, "null argument");
  int rc = decode_schedule(pool, seqs, n_seqs, 0, n_layers);
  if (rc) return rc;
  *bytes = pool->sched.total_bytes;
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_decode_plan_info(pkv_pool* pool, const pkv_seq* seqs, int32_t n_seqs, int32_t n_layers,
                         pkv_plan_info* info) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool) || !info) return fail(PKV_E_INVALID, "null argument");
  int rc = decode_schedule(pool, seqs, n_seqs, 0, n_layers);
  if (rc) return rc;
  const Schedule& S = pool->sched;
  info->n_segments = S.n_segments;
  info->n_chunks = S.n_chunks;
  info->n_items = (int32_t)S.items.size();
  info->partial_rows = S.P;
  info->unique_tokens = S.unique_tokens;
  info->wide_tokens = S.wide_tokens;
  info->workspace_bytes = (int64_t)S.total_bytes;
  info->plan_bytes = (int64_t)S.meta_bytes;
  info->read_tokens = S.tree ? S.unique_tokens : 0;
  info->grouped_items = 0;
  const int32_t bs = pool->pool.desc().block_size;
  for (const WorkItem& w : S.items) {
    info->read_tokens += (int64_t)(w.n_tok + bs - 1) / bs * bs;
    info->grouped_items += w.grouped ? 1 : 0;
  }
  info->reserved = 0;
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_decode_attn(pkv_pool* pool, const pkv_seq* seqs, int32_t n_seqs, int32_t layer0,
                    int32_t n_layers, const void* q, float* out, float scale, void* ws,
                    size_t ws_bytes, void* stream) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  const pkv_pool_desc& d = pool->pool.desc();
  if (!has_arenas(d)) return fail(PKV_E_INVALID, "pool has no device arenas");
  if (!q || !out) return fail(PKV_E_INVALID, "decode: null q or out");
  const bool mfma = use_mfma(pool);
  if (!attn_supported(mfma, d.kv_dtype, d.head_dim, d.block_size))
    return fail(PKV_E_UNSUPPORTED, "decode: head_dim must be 64/128/256 and block_size 16/32/64");
  // the workspace-size query plans layer0 = 0; the plan does not depend on it
  int rc = decode_schedule(pool, seqs, n_seqs, 0, n_layers);
  if (rc) return rc;
  if (layer0 < 0 || layer0 + n_layers > d.num_layers)
    return fail(PKV_E_INVALID, "decode: layer range outside the pool");
  return run_attention(pool, mfma, layer0, q, out, scale, ws, ws_bytes, (hipStream_t)stream);
  PKV_GUARD_END
}

int pkv_decode_attn_noalloc(pkv_pool* pool, const pkv_seq* seqs, int32_t n_seqs, int32_t layer0,
                            int32_t n_layers, const void* q, float* out, float scale, void* stream) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  const pkv_pool_desc& d = pool->pool.desc();
  if (!has_arenas(d)) return fail(PKV_E_INVALID, "pool has no device arenas");
  if (!q || !out) return fail(PKV_E_INVALID, "decode: null q or out");
  const bool mfma = use_mfma(pool);
  if (!attn_supported(mfma, d.kv_dtype, d.head_dim, d.block_size))
    return fail(PKV_E_UNSUPPORTED, "decode: head_dim must be 64/128/256 and block_size 16/32/64");
  int rc = decode_schedule(pool, seqs, n_seqs, 0, n_layers);
  if (rc) return rc;
  if (layer0 < 0 || layer0 + n_layers > d.num_layers)
    return fail(PKV_E_INVALID, "decode: layer range outside the pool");
  if (pool->sched.total_bytes > kScratchBytes)
    return fail(PKV_E_WORKSPACE, "decode_noalloc: the call needs " +
                                     std::to_string(pool->sched.total_bytes) +
                                     " bytes of workspace, more than the static scratch's " +
                                     std::to_string(kScratchBytes));
  void* ws = nullptr;
  hipError_t e = scratch_pointer(&ws);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  return run_attention(pool, mfma, layer0, q, out, scale, ws, kScratchBytes, (hipStream_t)stream,
                       true);
  PKV_GUARD_END
}

int pkv_verify_workspace_size(pkv_pool* pool, const pkv_seq* reqs, int32_t n_req, int32_t n_nodes,
                              size_t* bytes) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool) || !bytes) return fail(PKV_E_INVALID, "null argument");
  // the plan depends on the tree only through the masks, not on its sizes
  const size_t np = (size_t)(n_req > 0 ? n_req : 0) * (n_nodes > 0 ? n_nodes : 0);
  std::vector<int32_t> chain(np);
  for (size_t i = 0; i < np; ++i) chain[i] = (int32_t)(i % n_nodes) - 1;
  Schedule s;
  int rc = build_verify_schedule(pool->pool, reqs, n_req, chain.data(), n_nodes,
                                 planner_options(pool, true), &s);
  if (rc) return rc;
  *bytes = s.total_bytes;
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_tree_verify_attn(pkv_pool* pool, const pkv_seq* reqs, int32_t n_req, const int32_t* parents,
                         int32_t n_nodes, int32_t layer, const void* q, float* out, float scale,
                         void* ws, size_t ws_bytes, void* stream) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool)) return fail(PKV_E_INVALID, "null pool");
  const pkv_pool_desc& d = pool->pool.desc();
  if (!has_arenas(d)) return fail(PKV_E_INVALID, "pool has no device arenas");
  if (!q || !out) return fail(PKV_E_INVALID, "verify: null q or out");
  if (layer < 0 || layer >= d.num_layers) return fail(PKV_E_INVALID, "verify: layer outside the pool");
  if (!attn_supported(true, d.kv_dtype, d.head_dim, d.block_size))
    return fail(PKV_E_UNSUPPORTED, "verify: needs bf16 K/V, head_dim 64/128/256, block_size 16/32/64");
  int rc = verify_schedule(pool, reqs, n_req, parents, n_nodes);
  if (rc) return rc;
  return run_attention(pool, true, layer, q, out, scale, ws, ws_bytes, (hipStream_t)stream);
  PKV_GUARD_END
}

int pkv_pool_set_option(pkv_pool* pool, const char* key, int64_t value) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool) || !key) return fail(PKV_E_INVALID, "null argument");
  const std::string k(key);
  if (k == "path") {
    if (value < 0 || value > 2) return fail(PKV_E_INVALID, "path must be 0, 1 or 2");
    pool->path = (int)value;
  } else if (k == "chunk_tokens") {
    if (value < 0 || value > (1 << 24)) return fail(PKV_E_INVALID, "chunk_tokens out of range");
    pool->opt.chunk_tokens = (int32_t)value;
  } else if (k == "rows_per_item") {
    if (value < 1 || value > 64) return fail(PKV_E_INVALID, "rows_per_item must be 1..64");
    pool->opt.rows_per_item = (int32_t)value;
  } else if (k == "wide") {
    if (value < 0 || value > 1) return fail(PKV_E_INVALID, "wide must be 0 or 1");
    pool->opt.wide = value != 0;
  } else if (k == "prefetch") {
    if (value < 0 || value > 1) return fail(PKV_E_INVALID, "prefetch must be 0 or 1");
    pool->prefetch = (int)value;
  } else if (k == "short_tokens") {
    if (value < 32 || value > 8192) return fail(PKV_E_INVALID, "short_tokens must be 32..8192");
    pool->opt.short_tokens = (int32_t)value;
  } else if (k == "fold_tokens") {
    if (value < 0 || value > 8192) return fail(PKV_E_INVALID, "fold_tokens must be 0..8192");
    pool->opt.fold_tokens = (int32_t)value;
  } else if (k == "group_rows") {
    if (value < 0 || value > 16) return fail(PKV_E_INVALID, "group_rows must be 0..16");
    pool->opt.group_rows = (int32_t)value;
  } else if (k == "short_items") {
    if (value < 0 || value > 1) return fail(PKV_E_INVALID, "short_items must be 0 or 1");
    pool->opt.short_items = value != 0;
  } else if (k == "prefix_cache_blocks") {
    return pool->pool.set_prefix_capacity(value);
  } else if (k == "finalize") {
    if (value < 0 || value > 1) return fail(PKV_E_INVALID, "finalize must be 0 or 1");
    pool->opt.finalize = value != 0;
  } else if (k == "inline_plan") {
    if (value < 0 || value > 1) return fail(PKV_E_INVALID, "inline_plan must be 0 or 1");
    pool->inline_plan = (int)value;
  } else if (k == "concurrent") {
    if (value < 0 || value > 1) return fail(PKV_E_INVALID, "concurrent must be 0 or 1");
    pool->concurrent = (int)value;
  } else if (k == "row_blocks_per_wave") {
    if (value < 0 || value > 2) return fail(PKV_E_INVALID, "row_blocks_per_wave must be 0, 1 or 2");
    pool->opt.max_row_blocks_per_wave = (int32_t)value;
  } else if (k == "wide_waves") {
    if (value != 0 && value != 4 && value != 6 && value != 8)
      return fail(PKV_E_INVALID, "wide_waves must be 0 (automatic), 4, 6 or 8");
    pool->wide_waves = (int)value;
  } else if (k == "wide_row_blocks") {
    if (value < 0 || value > 2)
      return fail(PKV_E_INVALID, "wide_row_blocks must be 0 (automatic), 1 or 2");
    pool->wide_row_blocks = (int)value;
  } else if (k == "wide_spec") {
    if (value < 0 || value > 2) return fail(PKV_E_INVALID, "wide_spec must be 0, 1 or 2");
    pool->wide_spec = (int)value;
  } else if (k == "wide_fill") {
    if (value < 0 || value > 1) return fail(PKV_E_INVALID, "wide_fill must be 0 or 1");
    pool->opt.wide_fill = value != 0;
  } else if (k == "wide_rows") {
    if (value < 16 || value > 256) return fail(PKV_E_INVALID, "wide_rows must be 16..256");
    pool->opt.wide_rows = (int32_t)value;
  } else if (k == "tree") {
    if (value < 0 || value > 2) return fail(PKV_E_INVALID, "tree must be 0, 1 or 2");
    pool->opt.tree = (int32_t)value;
  } else if (k == "tree_stages") {
    if (value < 4 || value > 6) return fail(PKV_E_INVALID, "tree_stages must be 4, 5 or 6");
    pool->tree_stages = (int)value;
  } else if (k == "tree_piece_tokens") {
    if (value < 32 || value > 8192) return fail(PKV_E_INVALID, "tree_piece_tokens must be 32..8192");
    pool->opt.tree_piece_tokens = (int32_t)value;
  } else if (k == "timing") {
    if (value < 0 || value > 1) return fail(PKV_E_INVALID, "timing must be 0 or 1");
    pool->timing = value != 0;
  } else if (k == "tokens_per_row") {
    if (value < 0 || value > 8192) return fail(PKV_E_INVALID, "tokens_per_row must be 0..8192");
    pool->opt.tokens_per_row = (int32_t)value;
  } else if (k == "min_chunk_tokens") {
    if (value != 0 && (value < 32 || value > 8192))
      return fail(PKV_E_INVALID, "min_chunk_tokens must be 0 or 32..8192");
    pool->opt.min_chunk_tokens = (int32_t)value;
  } else if (k == "target_workgroups") {
    if (value < 1 || value > (1 << 24)) return fail(PKV_E_INVALID, "target_workgroups out of range");
    pool->opt.target_workgroups = (int32_t)value;
  } else {
    return fail(PKV_E_INVALID, "unknown option " + k);
  }
  pool->cache_valid = false;
  return PKV_OK;
  PKV_GUARD_END
}

int pkv_timing_read(pkv_pool* pool, const char* kernel, double* total_ms, int64_t* launches) {
  PKV_GUARD_BEGIN
  if (!pool_ok(pool) || !kernel || !total_ms || !launches) return fail(PKV_E_INVALID, "null argument");
  const std::string k(kernel);
  int kind = k == "attention" ? T_ATTN
             : k == "attention_wide" ? T_WIDE
             : k == "attention_span" ? T_SPAN
             : k == "combine" ? T_COMBINE
             : k == "append" ? T_APPEND
             : k == "commit_gather" ? T_GATHER
             : k == "attention_tree" ? T_TREE
                               : -1;
  if (kind < 0) return fail(PKV_E_INVALID, "unknown kernel " + k);
  return pool->timers[kind].read(total_ms, launches);
  PKV_GUARD_END
}

const char* pkv_last_error(void) { return last_error(); }

const char* pkv_version(void) { return "pkv 0.1.0 (gfx950)"; }

}  // extern "C"
