// Device kernels of the paged KV cache, written for gfx950 (MI355X, wave64).
//
//   append_kernel      copy-on-write copies and the scatter of appended
//                      tokens' K/V into their slots, in one launch
//   attn_mfma_kernel   paged attention over shared tiles on the matrix cores
//                      (bf16 K/V and q, fp32 softmax and accumulation); with a
//                      draft-tree mask it is the verify kernel
//   attn_valu_kernel   the same work on the vector ALUs (fp32 or bf16 K/V)
//   combine_kernel     log-sum-exp merge of a row's partial states in
//                      logical order
//
// Layout: K tiles [BS][D] (token-major), V tiles [D][BS] (token index
// fastest). See include/pkv.h.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kernel_common.h"
#include "kernels.hpp"

namespace pkv {

// ------------------------------------------------------------- append
//
// One launch performs an append's copy-on-write copies and its token writes.
// Workgroups [0, n_ops * L * Hkv) build the destination tile of one
// (op, layer, KV head): the source's slots [0, n_valid) plus the new tokens
// that land in the block (slots n_valid .. n_valid + m - 1); slots above
// that are left unspecified. V rows ([BS] per (head, d)) are copied whole
// with 16-byte vectors and patched in registers. No other workgroup writes
// the destination block. A copy's source is shared, so in general no write
// touches it; the one exception (after a truncate, a holder that sees fewer
// valid slots writes in place once the other holder's copy is planned) is
// split by the host into a copies-only launch followed by a writes-only
// launch, so within one launch copies and writes need no ordering. The
// remaining workgroups write one (layer, token) of the write list each, all
// KV heads. Copies are written with non-temporal stores: a decode usually
// follows, and with the copied tiles left in the caches the attention launch
// after the append ran ~2% slower (beam step: 97.9 -> 95.7 us with streaming
// stores). Their sources are read with non-temporal loads too (read once:
// append 9.65 -> 9.5 us).

template <typename T, int BS>
__device__ __forceinline__ void append_copy(const AppendParams& p, int o, int l, int h) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int RV = BS / EPV;  // 16-byte vectors per V row
  const int32_t* op = p.ops ? p.ops + 5 * o : p.inl_ops + 5 * o;
  const int src = op[0], dst = op[1], nv = op[2], tok0 = op[3], m = op[4];
  const int64_t tile = (int64_t)BS * p.D;
  T* __restrict__ K = (T*)p.k_arena;
  T* __restrict__ V = (T*)p.v_arena;
  const T* __restrict__ kn = (const T*)p.k_new;
  const T* __restrict__ vn = (const T*)p.v_new;
  const int64_t st = ((int64_t)l * p.NB + src) * p.Hkv + h;
  const int64_t dt = ((int64_t)l * p.NB + dst) * p.Hkv + h;
  // K rows: [0, nv) from the source, [nv, nv + m) from the new tokens
  const int vrow = p.D / EPV;  // vectors per K row
  for (int i = threadIdx.x; i < (nv + m) * vrow; i += blockDim.x) {
    const int t = i / vrow, c = i - t * vrow;
    const u32x4* from =
        t < nv ? (const u32x4*)(K + st * tile + (int64_t)t * p.D) + c
               : (const u32x4*)(kn + (((int64_t)l * p.n_tok + tok0 + t - nv) * p.Hkv + h) * p.D) + c;
    const u32x4 x = __builtin_nontemporal_load(from);
    __builtin_nontemporal_store(x, (u32x4*)(K + dt * tile + (int64_t)t * p.D) + c);
  }
  // V rows: whole rows from the source, new tokens patched in (slot k of
  // the row is visited with a compile-time index, so the row stays in
  // registers)
  typedef T vecT __attribute__((ext_vector_type(EPV)));
  for (int d = threadIdx.x; d < p.D; d += blockDim.x) {
    const vecT* vs = (const vecT*)(V + st * tile + (int64_t)d * BS);
    vecT row[RV];
#pragma unroll
    for (int c = 0; c < RV; ++c) row[c] = __builtin_nontemporal_load(vs + c);
    const T* vnew = vn + (((int64_t)l * p.n_tok + tok0) * p.Hkv + h) * p.D + d;
#pragma unroll
    for (int k = 0; k < BS; ++k)
      if (k >= nv && k < nv + m) row[k / EPV][k % EPV] = vnew[(int64_t)(k - nv) * p.Hkv * p.D];
    vecT* vd = (vecT*)(V + dt * tile + (int64_t)d * BS);
#pragma unroll
    for (int c = 0; c < RV; ++c) __builtin_nontemporal_store(row[c], vd + c);
  }
}

template <typename T, int BS>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int n_copy = p.n_ops * p.L * p.Hkv;
  if ((int)blockIdx.x < n_copy) {
    const int per_op = p.L * p.Hkv;
    const int o = blockIdx.x / per_op;
    const int r = blockIdx.x - o * per_op;
    append_copy<T, BS>(p, o, r / p.Hkv, r - (r / p.Hkv) * p.Hkv);
    return;
  }
  const int w = blockIdx.x - n_copy;  // (layer, write entry)
  const int l = w / p.n_write, i = w - l * p.n_write;
  const int64_t slot = p.wslots ? p.wslots[i] : p.inl_slots[i];
  const int tok = p.wtok ? p.wtok[i] : p.inl_tok[i];
  const int64_t b = slot / BS;
  const int off = (int)(slot - b * BS);
  const int64_t t0 = ((int64_t)l * p.NB + b) * p.Hkv;
  T* K = (T*)p.k_arena;
  T* V = (T*)p.v_arena;
  const T* kn = (const T*)p.k_new + ((int64_t)l * p.n_tok + tok) * p.Hkv * p.D;
  const T* vn = (const T*)p.v_new + ((int64_t)l * p.n_tok + tok) * p.Hkv * p.D;
  for (int e = threadIdx.x; e < p.Hkv * p.D; e += blockDim.x) {
    const int h = e / p.D, d = e - h * p.D;
    K[((t0 + h) * BS + off) * p.D + d] = kn[e];
    V[((t0 + h) * p.D + d) * BS + off] = vn[e];
  }
}

// ------------------------------------------------------------- gather
//
// One workgroup per (layer, token): the token's K rows (contiguous D per
// KV head) and V columns (stride BS in the d-major V tile) are copied into
// [L][n_rows][Hkv][D] outputs. Used to keep a verified draft path: its tokens
// are read out before the tree is truncated, then appended again.

template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(GatherParams p) {
  const int l = blockIdx.x / p.n, i = blockIdx.x - (blockIdx.x / p.n) * p.n;
  const int64_t slot = p.slots[i];
  const int64_t b = slot / p.BS;
  const int off = (int)(slot - b * p.BS);
  const int64_t t0 = ((int64_t)l * p.NB + b) * p.Hkv;
  const T* K = (const T*)p.k_arena;
  const T* V = (const T*)p.v_arena;
  T* ko = (T*)p.k_out + ((int64_t)l * p.n_rows + p.row0 + i) * p.Hkv * p.D;
  T* vo = (T*)p.v_out + ((int64_t)l * p.n_rows + p.row0 + i) * p.Hkv * p.D;
  for (int e = threadIdx.x; e < p.Hkv * p.D; e += blockDim.x) {
    const int h = e / p.D, d = e - h * p.D;
    ko[e] = K[((t0 + h) * p.BS + off) * p.D + d];
    vo[e] = V[((t0 + h) * p.D + d) * p.BS + off];
  }
}

// ----------------------------------------------------- MFMA attention
//
// One workgroup (4 waves) per (work item, layer, KV head). A work item is a
// chunk of up to a few thousand tokens and up to 64 query rows that all
// read it. Rows are packed 16 to a row block; a 32-token step is
//   S^T = K Q^T   (two 16x16x32 bf16 MFMAs per 32 d, token rows x query cols)
//   O^T += V^T P^T (one 16x16x32 MFMA per 16 d, split P = hi + lo in bf16)
// Operand lane layouts (16x16x32): lane l holds A[l%16][8(l/16)+e] and
// B[8(l/16)+e][l%16] for e = 0..7; the result C[4(l/16)+i][l%16], i = 0..3.
// The contraction index can be permuted freely as long as A and B agree,
// and the row order of a K tile too: row m of S^T tile tau is token
// 8(m/4) + 4 tau + m%4, so a lane's eight scores are tokens 8(l/16) .. +7 of
// its query row l%16 -- exactly the B operand P^T of the P.V product, with
// no data movement. V tiles are stored d-major ([D][BS]) so that the A
// operand V^T[d][8 tokens] is one 16-byte load.
// A workgroup with 1 or 2 row blocks gives the spare waves alternate steps
// of the chunk and merges their states through LDS at the end.

template <int D, int BS, bool LO, bool PF, int RW>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnCore p, PlanBytes plan_bytes) {
  const PlanArrays sp = plan_arrays(p, plan_bytes);
  constexpr int KS = D / 32;  // 32-wide k steps of Q.K
  constexpr int DB = D / 16;  // 16-wide d blocks of P.V
  constexpr int ACC_STRIDE = D + 4;
  constexpr int SLOTS = 3 * RW;
  static_assert(BS == 16 || BS == 32 || BS == 64, "block size");
  static_assert(RW == 1 || (RW == 2 && !PF), "row blocks per wave");
  __shared__ float mrg_m[SLOTS][16];
  __shared__ float mrg_l[SLOTS][16];
  __shared__ float mrg_acc[SLOTS][16 * ACC_STRIDE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  // long items: the workgroup serves one code; short items: each wave one
  // (the workgroup's mode is uniform: short items come last). A short-item
  // workgroup takes four planes (layer, KV head) of one item, or, when the
  // plan folded short shared edges into every leaf's item, four consecutive
  // items of one plane, a plane's workgroups dealt to one XCD in consecutive
  // rounds (workgroup w goes to XCD w % 8), so that the leaves meet their
  // shared edges in one L2 (MCTS leaves: 148 -> 141 us; four planes of one
  // item read adjacent tiles and stayed faster for unshared items, 95 us
  // against 96 for the beam).
  const bool solo = (int)blockIdx.x >= p.n_long_wgs;
  int code = (int)blockIdx.x;
  if (!solo && p.long_by_plane) {
    // long items of a folded plan, dealt the same way: a plane's items in
    // consecutive rounds of one XCD, so that items reading the same edges
    // meet them in its L2
    const int planes = p.n_layers * p.Hkv;
    const int n_li = p.n_long / planes;
    const int r = (int)blockIdx.x >> 3;
    const int grp = r / n_li, k = r - grp * n_li;
    const int plane = grp * 8 + ((int)blockIdx.x & 7);
    code = plane < planes ? k * planes + plane : p.n_codes;
  } else if (solo && !p.short_by_plane) {
    code = p.n_long + ((int)blockIdx.x - p.n_long_wgs) * 4 + wave;
  } else if (solo) {
    const int planes = p.n_layers * p.Hkv;
    const int n_short = (p.n_codes - p.n_long) / planes;
    const int wpp = (n_short + 3) >> 2;  // workgroups per plane
    const int w = (int)blockIdx.x - p.n_long_wgs;
    const int r = w >> 3;
    const int grp = r / wpp, k = r - grp * wpp;
    const int plane = grp * 8 + (w & 7);
    const int s_item = 4 * k + wave;
    code = (plane < planes && s_item < n_short) ? p.n_long + s_item * planes + plane : p.n_codes;
  }
  if (code >= p.n_codes) return;  // whole waves of a solo workgroup, or a padding workgroup
  const int per_item = p.n_layers * p.Hkv;
  const int item_idx = code / per_item;
  const int rem = code - item_idx * per_item;
  const int li = rem / p.Hkv;
  const int kvh = rem - li * p.Hkv;
  const int layer = p.layer0 + li;
  const WorkItem it = sp.items[item_idx];

  // row blocks of 16 rows; a wave owns RW consecutive blocks (a row group)
  const int RB = (it.n_rows + 15) >> 4;
  const int RG = (RB + RW - 1) / RW;
  const int RGp = RG == 1 ? 1 : (RG == 2 ? 2 : 4);
  const int phases = solo ? 1 : 4 / RGp;
  const int rg = solo ? 0 : wave % RGp, phase = solo ? 0 : wave / RGp;
  const bool active = rg < RG;
  const int nblk = active ? min(RW, RB - rg * RW) : 0;  // wave-uniform

  bf16x8 qv[RW][KS];
  bool row_ok[RW];
  uint64_t anc[RW];
  const bool tree = it.mask_from != 0x7fffffff && it.t0 + it.n_tok > it.mask_from;
  // A grouped item holds several sibling branches' blocks, each once; a
  // block's binfo word has bit h set when the item's holder h reads it and
  // its valid slots in bits 16 and up: row r sees a token when its holder's
  // bit is set and the token's slot is valid.
  const bool grouped = it.grouped != 0;
  const int32_t* binfo = sp.binfo + it.blk_off;
  int32_t hbit[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = (rg * RW + r) * 16 + n;
    row_ok[r] = r < nblk && row < it.n_rows;
    const int crow = it.r0 + row;
    const int hold = crow / p.G;
    const int gq = crow - hold * p.G;
    hbit[r] = grouped ? 1 << (hold & 31) : 0;
    const int branch = row_ok[r] ? sp.holders[it.hold_off + hold] : 0;
    const int qh = kvh * p.G + gq;
    const uint16_t* qp =
        (const uint16_t*)p.q + (((int64_t)li * p.n_branch + branch) * p.Hq + qh) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok[r]) raw = ld16(qp + 32 * ks);
      qv[r][ks] = as_bf16x8(raw);
    }
    anc[r] = (tree && row_ok[r]) ? sp.anc[branch] : ~0ull;
  }

  const uint16_t* K = (const uint16_t*)p.k_arena;
  const uint16_t* V = (const uint16_t*)p.v_arena;
  const int64_t layer_tiles = (int64_t)layer * p.num_blocks * p.Hkv;
  const int32_t* blk = sp.blk + it.blk_off;

  // this lane's token offsets inside a 32-token step: K tile rows and V
  // columns; with 16-token blocks a step spans two blocks (A, B)
  const int koff0 = 8 * (n >> 2) + (n & 3);  // tile 0; tile 1 is +4
  const bool k_in_b = BS == 16 && koff0 >= 16;
  const int voff = 8 * g;
  const bool v_in_b = BS == 16 && voff >= 16;

  f32x4 acc[RW][DB];
  float m_run[RW], l_run[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
#pragma unroll
    for (int j = 0; j < DB; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[r] = kNegInf;
    l_run[r] = 0.f;
  }
  const int n_steps = (it.n_tok + 31) >> 5;
  // With prefetch the block ids come from LDS (see stage_block_ids); a
  // wave that loads one step at a time reads them from global memory one
  // step ahead (at D = 256 through the scalar cache), which spares short
  // items the staging round trip.
  __shared__ int32_t blk_s[PF ? kMaxChunkBlocks : 1];
  const bool staged = PF && !solo;  // (a solo wave reads its own ids)
  if (staged) {
    stage_block_ids<BS>(blk_s, blk, n_steps);
    __syncthreads();
  }

  // K rows of this lane (both S^T tiles) and V^T columns of step s
  const bool stream_kv = it.reread == 0;
  auto ldkv = [&](const uint16_t* ptr) { return stream_kv ? ld16_stream(ptr) : ld16(ptr); };
  auto load_k = [&](int s, int bA, int bB, u32x4 (&kr)[2][KS]) {
    const int kb = k_in_b ? bB : bA;
    const uint16_t* kp =
        K + ((layer_tiles + (int64_t)kb * p.Hkv + kvh) * BS + (s * 32 + koff0) % BS) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kr[0][ks] = ldkv(kp + 32 * ks);
      kr[1][ks] = ldkv(kp + 4 * D + 32 * ks);
    }
  };
  auto load_v = [&](int s, int bA, int bB, u32x4 (&vr)[DB]) {
    const int vb = v_in_b ? bB : bA;
    const uint16_t* vp =
        V + ((layer_tiles + (int64_t)vb * p.Hkv + kvh) * D + n) * BS + (s * 32 + voff) % BS;
#pragma unroll
    for (int j = 0; j < DB; ++j) vr[j] = ldkv(vp + (int64_t)16 * j * BS);
  };
  auto load_kv = [&](int s, int bA, int bB, u32x4 (&kr)[2][KS], u32x4 (&vr)[DB]) {
    load_k(s, bA, bB, kr);
    load_v(s, bA, bB, vr);
  };
  // binfo words of step s's two block slots (as ids reads the block ids;
  // the same word twice when a block spans the step)
  auto infos = [&](int s, int& a, int& b) {
    a = b = 0;
    if (grouped) {
      a = binfo[(32 * s) / BS];
      b = binfo[(32 * s + 16) / BS];
    }
  };
  // slots past the chunk may hold anything (even NaN): zero them in the
  // chunk's last step so that 0 * V stays 0 in the P.V product (in a
  // grouped item, the slots past each block's valid ones)
  auto zero_tail = [&](int s, u32x4 (&vraw)[DB], int iA, int iB) {
    const int tv = s * 32 + voff;
    int lim = it.n_tok;
    bool cut = s * 32 + 32 > it.n_tok;
    if (grouped && ((iA >> 16) < BS || (iB >> 16) < BS)) {
      lim = (tv & ~(BS - 1)) + ((v_in_b ? iB : iA) >> 16);
      cut = true;
    }
    if (cut) {
      u32x4 keep;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = (tv + 2 * w < lim) ? 0x0000ffffu : 0u;
        const uint32_t hi = (tv + 2 * w + 1 < lim) ? 0xffff0000u : 0u;
        keep[w] = lo | hi;
      }
#pragma unroll
      for (int j = 0; j < DB; ++j) vraw[j] &= keep;
    }
  };
  // the two S^T tiles of row block r
  auto scores_rb = [&](int r, const u32x4 (&kraw)[2][KS], f32x4 (&st)[2]) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) c = mfma_bf16(as_bf16x8(kraw[tau][ks]), qv[r][ks], c);
      st[tau] = c;
    }
  };
  // online softmax of row block r in step s, and its P.V products
  auto softmax_pv_rb = [&](int s, int r, const f32x4 (&st)[2], const u32x4 (&vraw)[DB], int iA,
                           int iB) {
    const int tbase = s * 32;
    const int tv = tbase + voff;
    // tokens at or past lim are masked: the chunk's end, or in a grouped
    // item the end of the valid slots of the lane's block when the row's
    // holder reads it, else the block's start (none); a step whose blocks
    // every holder reads in full needs no mask
    int lim = it.n_tok;
    bool cut = tbase + 32 > it.n_tok;
    if (grouped && ((iA & iB & 0xffff) != it.grouped || (iA >> 16) < BS || (iB >> 16) < BS)) {
      const int info = v_in_b ? iB : iA;
      lim = (tv & ~(BS - 1)) + ((info & hbit[r]) ? (info >> 16) : 0);
      cut = true;
    }
    float sc[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * tau + i;
        const int t = tv + e;
        float v = st[tau][i] * p.scale_log2;
        if (cut && t >= lim) v = kNegInf;
        if (tree) {
          const int pos = it.t0 + t;
          if (pos >= it.mask_from && !((anc[r] >> (pos - it.mask_from)) & 1ull)) v = kNegInf;
        }
        sc[e] = v;
      }
    const float mx = max_xor32(max_xor16(rmax8(sc)));
    rebase(mx, m_run[r], l_run[r], acc[r]);
    const float m_use = (m_run[r] == kNegInf) ? 0.f : m_run[r];
    float psum = 0.f;
    bf16x8 phi, plo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = fast_exp2(sc[e] - m_use);
      psum += pe;
      const __bf16 h = (__bf16)pe;
      phi[e] = h;
      if (LO) plo[e] = (__bf16)(pe - (float)h);
    }
    l_run[r] += psum;
#pragma unroll
    for (int j = 0; j < DB; ++j) {
      acc[r][j] = mfma_bf16(as_bf16x8(vraw[j]), phi, acc[r][j]);
      if (LO) acc[r][j] = mfma_bf16(as_bf16x8(vraw[j]), plo, acc[r][j]);
    }
  };
  auto compute = [&](int s, const u32x4 (&kraw)[2][KS], u32x4 (&vraw)[DB], int iA, int iB) {
    zero_tail(s, vraw, iA, iB);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (r > 0 && r >= nblk) continue;
      f32x4 st[2];
      scores_rb(r, kraw, st);
      softmax_pv_rb(s, r, st, vraw, iA, iB);
      // one row block at a time: interleaving the two would keep both
      // blocks' scores and probabilities live
      if (RW > 1) __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (active && phase < n_steps) {
    auto ids = [&](int s, int& a, int& b) {
      // (a branch, not a pointer select: LDS and global reads stay apart)
      if (staged) {
        a = blk_s[(32 * s) / BS];
        b = blk_s[(32 * s + 16) / BS];
      } else {
        a = blk[(32 * s) / BS];
        b = blk[(32 * s + 16) / BS];
      }
    };
    if (!PF && D <= 128) {
      int bA, bB, iA, iB;
      ids(phase, bA, bB);
      infos(phase, iA, iB);
      for (int s = phase; s < n_steps; s += phases) {
        const int cA = bA, cB = bB, jA = iA, jB = iB;
        if (s + phases < n_steps) {
          ids(s + phases, bA, bB);
          infos(s + phases, iA, iB);
        }
        u32x4 kr[2][KS], vr[DB];
        load_kv(s, cA, cB, kr, vr);
        compute(s, kr, vr, jA, jB);
      }
    } else if (!PF) {
      // D = 256 (one wave per SIMD, a 32 KiB step per wave): one register
      // set, refilled as it frees: the K tiles of the wave's
      // next step are loaded as soon as this step's scores are taken, its V
      // tiles as soon as this step's P.V is done, so that one step of K/V
      // stays in flight through the math. The last step is peeled off, so
      // every load in the loop is unconditional and the compiler's waits
      // count exactly the younger loads. Block ids are read through the
      // scalar cache (waited on with the LDS counter, so the wait does not
      // drain the K/V loads in flight). Measured: agent decode 125 -> 121 us;
      // at D = 128 the plain loop above was ~4% faster (beam decode).
      typedef const __attribute__((address_space(4))) int32_t* ids_ptr;
      const ids_ptr cblk = (ids_ptr)blk;
      const int last = n_steps - 1;
      const int s1 = min(phase + phases, last);
      int bA = cblk[(32 * phase) / BS], bB = cblk[(32 * phase + 16) / BS];
      int nA = cblk[(32 * s1) / BS], nB = cblk[(32 * s1 + 16) / BS];
      u32x4 kr[2][KS], vr[DB];
      load_kv(phase, bA, bB, kr, vr);
      int s = phase;
      for (; s + phases < n_steps; s += phases) {
        const int sn = s + phases;
        bA = nA;
        bB = nB;
        const int s2 = min(sn + phases, last);
        nA = cblk[(32 * s2) / BS];
        nB = cblk[(32 * s2 + 16) / BS];
        f32x4 st[RW][2];
#pragma unroll
        for (int r = 0; r < RW; ++r)
          if (r == 0 || r < nblk) scores_rb(r, kr, st[r]);
        __builtin_amdgcn_sched_barrier(0);
        load_k(sn, bA, bB, kr);
        __builtin_amdgcn_sched_barrier(0);
        int iA, iB;
        infos(s, iA, iB);
        zero_tail(s, vr, iA, iB);
#pragma unroll
        for (int r = 0; r < RW; ++r)
          if (r == 0 || r < nblk) softmax_pv_rb(s, r, st[r], vr, iA, iB);
        __builtin_amdgcn_sched_barrier(0);
        load_v(sn, bA, bB, vr);
        __builtin_amdgcn_sched_barrier(0);
      }
      int iA, iB;
      infos(s, iA, iB);
      compute(s, kr, vr, iA, iB);
    } else {
      // loads of the wave's next step are in flight while this one computes
      // (two register sets, loop unrolled by two)
      // (the prefetch is unconditional, re-reading the last step past the
      // end, so that the compiler's wait before each step's math counts
      // only that step's loads)
      const int last = n_steps - 1;
      u32x4 ka[2][KS], va[DB], kb[2][KS], vb[DB];
      int bA, bB;
      ids(phase, bA, bB);
      load_kv(phase, bA, bB, ka, va);
      for (int s = phase; s < n_steps; s += 2 * phases) {
        const int s1 = s + phases;
        ids(min(s1, last), bA, bB);
        load_kv(min(s1, last), bA, bB, kb, vb);
        __builtin_amdgcn_sched_barrier(0);
        int iA, iB;
        infos(s, iA, iB);
        compute(s, ka, va, iA, iB);
        if (s1 >= n_steps) break;
        const int s2 = min(s1 + phases, last);
        ids(s2, bA, bB);
        load_kv(s2, bA, bB, ka, va);
        __builtin_amdgcn_sched_barrier(0);
        infos(s1, iA, iB);
        compute(s1, kb, vb, iA, iB);
      }
    }
  }
  // the four lane groups hold disjoint tokens of the same rows
  float l_fin[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) l_fin[r] = sum_xor32(sum_xor16(l_run[r]));

  if (phases > 1) {
    if (phase > 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        if (r > 0 && r >= nblk) continue;
        const int slot = ((phase - 1) * RGp + rg) * RW + r;
        if (g == 0) {
          mrg_m[slot][n] = m_run[r];
          mrg_l[slot][n] = l_fin[r];
        }
#pragma unroll
        for (int j = 0; j < DB; ++j)
          *(f32x4*)&mrg_acc[slot][n * ACC_STRIDE + 16 * j + 4 * g] = acc[r][j];
      }
    }
    __syncthreads();
    if (phase == 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        if (r > 0 && r >= nblk) continue;
        for (int ph = 1; ph < phases; ++ph) {
          const int slot = ((ph - 1) * RGp + rg) * RW + r;
          const float mo = mrg_m[slot][n], lo = mrg_l[slot][n];
          const float M = fmaxf(m_run[r], mo);
          if (M != kNegInf) {
            const float a = fast_exp2(m_run[r] - M), b = fast_exp2(mo - M);
            l_fin[r] = l_fin[r] * a + lo * b;
#pragma unroll
            for (int j = 0; j < DB; ++j) {
              const f32x4 o = *(const f32x4*)&mrg_acc[slot][n * ACC_STRIDE + 16 * j + 4 * g];
              acc[r][j] = acc[r][j] * a + o * b;
            }
            m_run[r] = M;
          }
        }
      }
    }
  }
  if (phase == 0) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (!row_ok[r]) continue;
      const int row = (rg * RW + r) * 16 + n;
      if (p.finalize) {
        // the branch's other partial states (written by the wide launch,
        // which ran first) merged with this row's, in the combine's order
        // and arithmetic: per batch of eight, the batch maximum first, then
        // the entries in logical order; the output row is written here
        const int crow = it.r0 + row;
        const int hold = crow / p.G;
        const int gq = crow - hold * p.G;
        const int branch = sp.holders[it.hold_off + hold];
        const int64_t pl = (int64_t)(li * p.Hkv + kvh) * p.P;
        const int own = it.part_row + row;
        const int e0 = sp.comb_ptr[branch], e1 = sp.comb_ptr[branch + 1];
        float M = kNegInf, L = 0.f;
        f32x4 o[DB];
#pragma unroll
        for (int j = 0; j < DB; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int e = e0; e < e1; e += 8) {
          const int ne = min(8, e1 - e);
          float bm = kNegInf;
          for (int k = 0; k < ne; ++k) {
            const int rk = sp.comb_rows[e + k] + gq;
            bm = fmaxf(bm, rk == own ? m_run[r] : p.part_ml[2 * (pl + rk)]);
          }
          const float Mn = fmaxf(M, bm);
          if (Mn == kNegInf) continue;
          const float a = M == kNegInf ? 0.f : fast_exp2(M - Mn);
          L *= a;
#pragma unroll
          for (int j = 0; j < DB; ++j) o[j] *= a;
          for (int k = 0; k < ne; ++k) {
            const int rk = sp.comb_rows[e + k] + gq;
            const bool mine = rk == own;
            const float mk = mine ? m_run[r] : p.part_ml[2 * (pl + rk)];
            const float lk = mine ? l_fin[r] : p.part_ml[2 * (pl + rk) + 1];
            const float wk = mk == kNegInf ? 0.f : fast_exp2(mk - Mn);
            L += lk * wk;
            const float* pa = p.part_acc + (pl + rk) * D;
#pragma unroll
            for (int j = 0; j < DB; ++j)
              o[j] += (mine ? acc[r][j] : *(const f32x4*)(pa + 16 * j + 4 * g)) * wk;
          }
          M = Mn;
        }
        float* orow = p.out + (((int64_t)li * p.n_branch + branch) * p.Hq + kvh * p.G + gq) * D;
#pragma unroll
        for (int j = 0; j < DB; ++j) *(f32x4*)(orow + 16 * j + 4 * g) = o[j] / L;
        continue;
      }
      const int64_t prow = (int64_t)(li * p.Hkv + kvh) * p.P + it.part_row + row;
      if (g == 0) {
        p.part_ml[2 * prow] = m_run[r];
        p.part_ml[2 * prow + 1] = l_fin[r];
      }
      float* pa = p.part_acc + prow * D;
#pragma unroll
      for (int j = 0; j < DB; ++j) *(f32x4*)(pa + 16 * j + 4 * g) = acc[r][j];
    }
  }
}

// ------------------------------------------------- wide MFMA attention
//
// For chunks read by many query rows (draft-tree verify: nodes x GQA group;
// the shared root of a wide tree). One workgroup serves up to 16 * NC * RBW
// rows with NC compute waves (wave w owns row blocks w + NC * r, r < RBW)
// and NP loader waves. Each 32-token step of K/V is loaded once for the
// whole workgroup straight from global memory into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at l * 16 of a 1 KiB
// section), already in operand order: one section per (K tile, k step) and
// per V d block, so every operand read is a conflict-free ds_read_b128 and
// each compute wave applies it to all of its row blocks. The loader waves
// keep two steps in flight in a ring of three LDS stages; they never read
// LDS and the compute waves never load from global memory, so neither
// waits on the other's traffic beyond the one barrier per step. Math per
// row block is the narrow kernel's.

template <int D>
constexpr int wide_loaders() { return D == 256 ? 2 : 1; }

template <int D, int BS, int NC, int RBW>
__global__ __launch_bounds__((NC + wide_loaders<D>()) * 64) void attn_wide_kernel(AttnCore p, PlanBytes plan_bytes) {
  const PlanArrays sp = plan_arrays(p, plan_bytes);
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  constexpr int NP = wide_loaders<D>();
  constexpr int NSEC = 2 * KS + DB;  // 1 KiB sections per step
  constexpr int SPL = NSEC / NP;     // sections per loader wave per step
  static_assert(NSEC % NP == 0 && 2 * SPL < 64, "loads in flight per loader wave");
  static_assert(BS == 16 || BS == 32 || BS == 64, "block size");
  static_assert(RBW == 1 || RBW == 2, "row blocks per wave");
  // the ring's stages as separate arrays
  __shared__ u32x4 st0[NSEC * 64], st1[NSEC * 64], st2[NSEC * 64];
  __shared__ int32_t blk_s[kMaxChunkBlocks];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool loader = wave >= NC;
  const int n = lane & 15, g = lane >> 4;
  const int code = sp.order[blockIdx.x];
  if (code < 0) return;
  const int per_item = p.n_layers * p.Hkv;
  const int item_idx = code / per_item;
  const int rem = code - item_idx * per_item;
  const int li = rem / p.Hkv;
  const int kvh = rem - li * p.Hkv;
  const int layer = p.layer0 + li;
  const WorkItem it = sp.items[item_idx];
  const int n_steps = (it.n_tok + 31) >> 5;
  const int last = n_steps - 1;
  stage_block_ids<BS>(blk_s, sp.blk + it.blk_off, n_steps);
  __syncthreads();
  const int voff = 8 * g;

  // One barrier per step; the s_waitcnt immediate below has vmcnt in bits
  // 3:0 and 15:14, expcnt 7 and lgkmcnt 15 meaning "no wait" on those. The
  // barrier is the bare s_barrier: a workgroup fence would make every wave
  // wait for all of its loads in flight.
  if (loader) {
    const int lw = wave - NC;
    const uint16_t* K = (const uint16_t*)p.k_arena;
    const uint16_t* V = (const uint16_t*)p.v_arena;
    const int64_t layer_tiles = (int64_t)layer * p.num_blocks * p.Hkv;
    const int koff0 = 8 * (n >> 2) + (n & 3);
    // sections lw + NP * i of step s (the first 2KS are K, the rest V)
    auto issue = [&](int s, u32x4* buf) __attribute__((always_inline)) {
      const int tbase = 32 * s;
      const int bA = blk_s[tbase / BS];
      const int bB = blk_s[(tbase + 16) / BS];
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int sect = lw + NP * i;
        const uint16_t* src;
        if (sect < 2 * KS) {
          const int tau = sect / KS, ks = sect - (sect / KS) * KS;
          const int off = koff0 + 4 * tau;
          const int b = (BS == 16 && off >= 16) ? bB : bA;
          src = K + ((layer_tiles + (int64_t)b * p.Hkv + kvh) * BS + (tbase + off) % BS) * D +
                32 * ks + 8 * g;
        } else {
          const int j = sect - 2 * KS;
          const int b = (BS == 16 && voff >= 16) ? bB : bA;
          src = V + ((layer_tiles + (int64_t)b * p.Hkv + kvh) * D + 16 * j + n) * BS +
                (tbase + voff) % BS;
        }
        __builtin_amdgcn_global_load_lds(
            src, (__attribute__((address_space(3))) void*)&buf[sect * 64], 16, 0, 0);
      }
    };
    // At step s: wait for this wave's loads of step s (step s + 1's may
    // stay in flight), barrier (step s has landed everywhere and every
    // compute wave is done with step s - 1's stage), then load step s + 2
    // into that stage. Past the end the last step is loaded again (in
    // bounds, never read), so the count of younger loads is always SPL.
    // In the chunk's last step the V slots past its end may hold anything
    // (even NaN); each loader zeroes them in the V sections it loaded,
    // after they land and before the barrier, so that 0 * V stays 0.
    const bool ragged = (it.n_tok & 31) != 0;
    auto zero_tail = [&](u32x4* cur) __attribute__((always_inline)) {
      const int tv = 32 * last + voff;
      u32x4 keep;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = (tv + 2 * w < it.n_tok) ? 0x0000ffffu : 0u;
        const uint32_t hi = (tv + 2 * w + 1 < it.n_tok) ? 0xffff0000u : 0u;
        keep[w] = lo | hi;
      }
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int sect = lw + NP * i;
        if (sect >= 2 * KS) cur[sect * 64 + lane] &= keep;
      }
    };
    constexpr int kWaitVm = 0x0F70 | (SPL & 0xF) | ((SPL >> 4) << 14);
    auto step = [&](int s, u32x4* cur, u32x4* next) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(kWaitVm);
      if (ragged && s == last) zero_tail(cur);
      __builtin_amdgcn_s_barrier();
      issue(min(s + 2, last), next);
    };
    issue(0, st0);
    issue(min(1, last), st1);
    for (int s = 0; s < n_steps; s += 3) {
      step(s, st0, st2);
      if (s + 1 >= n_steps) break;
      step(s + 1, st1, st0);
      if (s + 2 >= n_steps) break;
      step(s + 2, st2, st1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    return;
  }

  const int RB = (it.n_rows + 15) >> 4;
  int nrb = 0;
#pragma unroll
  for (int r = 0; r < RBW; ++r) nrb += (wave + NC * r < RB) ? 1 : 0;
  const bool tree = it.mask_from != 0x7fffffff && it.t0 + it.n_tok > it.mask_from;

  bf16x8 qv[RBW][KS];
  bool row_ok[RBW];
  uint64_t anc[RBW];
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    const int row = (wave + NC * r) * 16 + n;
    row_ok[r] = r < nrb && row < it.n_rows;
    const int crow = it.r0 + row;
    const int hold = crow / p.G;
    const int gq = crow - hold * p.G;
    const int branch = row_ok[r] ? sp.holders[it.hold_off + hold] : 0;
    const uint16_t* qp = (const uint16_t*)p.q +
                         (((int64_t)li * p.n_branch + branch) * p.Hq + kvh * p.G + gq) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok[r]) raw = ld16(qp + 32 * ks) ^ p.q_flip;
      qv[r][ks] = as_bf16x8(raw);
    }
    anc[r] = (tree && row_ok[r]) ? sp.anc[branch] : ~0ull;
  }

  // acc[r][DB] holds the row sums: the products of P against a ones
  // operand (every output row of such a product is the row sum of P), so
  // the softmax adds no probabilities itself and the lazy rescale covers
  // the sums with the accumulators
  f32x4 acc[RBW][DB + 1];
#pragma unroll
  for (int r = 0; r < RBW; ++r)
#pragma unroll
    for (int j = 0; j <= DB; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[RBW], l_unused[RBW];
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    m_run[r] = kNegInf;
    l_unused[r] = 0.f;
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.f;
  // The row maximum across a row's four lanes is needed only when the
  // reference moves: when some lane's own maximum passes it by more than 8
  // (and on a row's first finite scores, where it is -inf).
  auto reference = [&](const float (&sc)[8], int r) __attribute__((always_inline)) {
    const float mxl = rmax8_fresh(sc) * p.abs_scale_log2;
    if (__any(mxl > m_run[r] + 8.f))
      rebase(max_xor32(max_xor16(mxl)), m_run[r], l_unused[r], acc[r]);
  };

  // Every row block of the wave is computed, also one past the item's last
  // (its query is zero and its state is never stored): a guard per product
  // splits the code into blocks that each wait for their own LDS read.
  auto compute_rb2 = [&](int step, const u32x4* st_sec) __attribute__((always_inline)) {
    const int s = step;
    if (nrb > 0) {
      f32x4 sc4[RBW][2];
#pragma unroll
      for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) sc4[r][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = as_bf16x8(st_sec[(tau * KS + ks) * 64 + lane]);
#pragma unroll
          for (int r = 0; r < RBW; ++r)
            sc4[r][tau] = mfma_bf16(a, qv[r][ks], sc4[r][tau]);
        }
      const int tbase = 32 * s;
      const bool tail = tbase + 32 > it.n_tok;
      const int tv = tbase + voff;
      bf16x8 phi[RBW], plo[RBW];
#pragma unroll
      for (int r = 0; r < RBW; ++r) {
        float sc[8];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[4 * tau + i] = sc4[r][tau][i];
        if (tail || tree) {  // wave-uniform: only the chunk's last step and masked steps
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = tv + e;
            if (t >= it.n_tok) sc[e] = kNegInf;
            const int pos = it.t0 + t;
            if (tree && pos >= it.mask_from && !((anc[r] >> (pos - it.mask_from)) & 1ull))
              sc[e] = kNegInf;
          }
        }
        reference(sc, r);
        const float m_use = (m_run[r] == kNegInf) ? 0.f : m_run[r];
        (void)probs8<true>(sc, p.abs_scale_log2, m_use, phi[r], plo[r]);
      }
#pragma unroll
      for (int j = 0; j < DB; ++j) {
        const bf16x8 a = as_bf16x8(st_sec[(2 * KS + j) * 64 + lane]);
#pragma unroll
        for (int r = 0; r < RBW; ++r) {
          acc[r][j] = mfma_bf16(a, phi[r], acc[r][j]);
          acc[r][j] = mfma_bf16(a, plo[r], acc[r][j]);
        }
      }
#pragma unroll
      for (int r = 0; r < RBW; ++r) {
        acc[r][DB] = mfma_bf16(ones, phi[r], acc[r][DB]);
        acc[r][DB] = mfma_bf16(ones, plo[r], acc[r][DB]);
      }
    }
  };
  // One row block per wave: operand reads from LDS run ahead of the
  // products in register rings (the compiler, left alone, waits for each
  // ds_read right before its product): K sections QD ahead during Q.K, and
  // the first VD V sections are issued before the softmax so that their
  // latency hides under it. (Two row blocks per wave leave no registers for
  // the rings; that form keeps the compiler's schedule.)
  constexpr int NK = 2 * KS;
  constexpr int QD = NK < 8 ? NK : 8;
  constexpr int VD = DB < 8 ? DB : 8;
  auto compute_rb1 = [&](int step, const u32x4* st_sec) __attribute__((always_inline)) {
    const int s = step;
    if (nrb > 0) {
      f32x4 sc4[RBW][2];
#pragma unroll
      for (int r = 0; r < RBW; ++r)
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) sc4[r][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
      // K sections in the order (ks, tau): consecutive products alternate
      // between the two score tiles
      auto ksec = [](int i) { return (i & 1) * KS + (i >> 1); };
      u32x4 kring[QD];
#pragma unroll
      for (int i = 0; i < QD; ++i) kring[i] = st_sec[ksec(i) * 64 + lane];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const bf16x8 a = as_bf16x8(kring[i % QD]);
        if (i + QD < NK) kring[i % QD] = st_sec[ksec(i + QD) * 64 + lane];
        const int tau = i & 1, ks = i >> 1;
#pragma unroll
        for (int r = 0; r < RBW; ++r) sc4[r][tau] = mfma_bf16(a, qv[r][ks], sc4[r][tau]);
        if (i + QD < NK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, RBW, 0);
      }
      u32x4 vring[VD];
#pragma unroll
      for (int i = 0; i < VD; ++i) vring[i] = st_sec[(2 * KS + i) * 64 + lane];
      __builtin_amdgcn_sched_barrier(0);
      const int tbase = 32 * s;
      const bool tail = tbase + 32 > it.n_tok;
      const int tv = tbase + voff;
      bf16x8 phi[RBW], plo[RBW];
#pragma unroll
      for (int r = 0; r < RBW; ++r) {
        float sc[8];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[4 * tau + i] = sc4[r][tau][i];
        if (tail || tree) {  // wave-uniform: only the chunk's last step and masked steps
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = tv + e;
            if (t >= it.n_tok) sc[e] = kNegInf;
            const int pos = it.t0 + t;
            if (tree && pos >= it.mask_from && !((anc[r] >> (pos - it.mask_from)) & 1ull))
              sc[e] = kNegInf;
          }
        }
        reference(sc, r);
        const float m_use = (m_run[r] == kNegInf) ? 0.f : m_run[r];
        (void)probs8<true>(sc, p.abs_scale_log2, m_use, phi[r], plo[r]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < DB; ++j) {
        const bf16x8 a = as_bf16x8(vring[j % VD]);
        if (j + VD < DB) vring[j % VD] = st_sec[(2 * KS + j + VD) * 64 + lane];
#pragma unroll
        for (int r = 0; r < RBW; ++r) {
          acc[r][j] = mfma_bf16(a, phi[r], acc[r][j]);
          acc[r][j] = mfma_bf16(a, plo[r], acc[r][j]);
        }
        if (j + VD < DB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * RBW, 0);
      }
#pragma unroll
      for (int r = 0; r < RBW; ++r) {
        acc[r][DB] = mfma_bf16(ones, phi[r], acc[r][DB]);
        acc[r][DB] = mfma_bf16(ones, plo[r], acc[r][DB]);
      }
    }
  };
  auto compute = [&](int step, const u32x4* st_sec) __attribute__((always_inline)) {
    if constexpr (RBW == 1)
      compute_rb1(step, st_sec);
    else
      compute_rb2(step, st_sec);
  };
  for (int s = 0; s < n_steps; s += 3) {
    __builtin_amdgcn_s_barrier();
    compute(s, st0);
    if (s + 1 >= n_steps) break;
    __builtin_amdgcn_s_barrier();
    compute(s + 1, st1);
    if (s + 2 >= n_steps) break;
    __builtin_amdgcn_s_barrier();
    compute(s + 2, st2);
  }

#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    if (r >= nrb) continue;
    const float l_tot = acc[r][DB][0];
    if (!row_ok[r]) continue;
    const int row = (wave + NC * r) * 16 + n;
    const int64_t prow = (int64_t)(li * p.Hkv + kvh) * p.P + it.part_row + row;
    if (g == 0) {
      p.part_ml[2 * prow] = m_run[r];
      p.part_ml[2 * prow + 1] = l_tot;
    }
    float* pa = p.part_acc + prow * D;
#pragma unroll
    for (int j = 0; j < DB; ++j) *(f32x4*)(pa + 16 * j + 4 * g) = acc[r][j];
  }
}

// ----------------------------------------------------- VALU attention
//
// One workgroup (4 waves) per (work item, layer, KV head), at most 16 rows.
// Each wave takes every fourth block of the chunk. Scores: lane
// (part, t) = (lane / BS, lane % BS) dots token t of the block with its
// 1/(64/BS) share of every query row (q staged in LDS as fp32), then the
// parts are summed with lane shuffles. P.V: lane owns d = lane + 64 k and
// reads the V^T row d of the block (BS contiguous values); the block's
// probabilities are broadcast through LDS.

template <typename T, int D, int BS>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnCore p, PlanBytes plan_bytes) {
  const PlanArrays sp = plan_arrays(p, plan_bytes);
  constexpr int LPT = 64 / BS;  // lanes per token in the score phase
  constexpr int DPL = D / LPT;  // d per lane in the score phase
  constexpr int DK = D / 64;    // d per lane in the P.V phase
  constexpr int MAXR = 16;
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte load
  static_assert(DPL % EPV == 0 && BS % EPV == 0, "vector width");
  __shared__ float qs[MAXR][D];
  __shared__ float ps[4][MAXR][BS];
  __shared__ float mrg_m[3][MAXR], mrg_l[3][MAXR];
  __shared__ float mrg_acc[3][MAXR][D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int code = blockIdx.x;  // (the vector-ALU plans have no short items)
  const int per_item = p.n_layers * p.Hkv;
  const int item_idx = code / per_item;
  const int rem = code - item_idx * per_item;
  const int li = rem / p.Hkv;
  const int kvh = rem - li * p.Hkv;
  const int layer = p.layer0 + li;
  const WorkItem it = sp.items[item_idx];
  const int nr = it.n_rows;

  const T* Q = (const T*)p.q;
  for (int idx = threadIdx.x; idx < nr * D; idx += blockDim.x) {
    const int r = idx / D, d = idx - (idx / D) * D;
    const int crow = it.r0 + r;
    const int hold = crow / p.G, gq = crow - (crow / p.G) * p.G;
    const int branch = sp.holders[it.hold_off + hold];
    qs[r][d] = to_f32<T>(Q[(((int64_t)li * p.n_branch + branch) * p.Hq + kvh * p.G + gq) * D + d]);
  }
  __syncthreads();

  const T* K = (const T*)p.k_arena;
  const T* V = (const T*)p.v_arena;
  const int64_t layer_tiles = (int64_t)layer * p.num_blocks * p.Hkv;
  const int32_t* blk = sp.blk + it.blk_off;
  const int t = lane % BS, part = lane / BS;

  float acc[MAXR][DK];
  float m[MAXR], lsum[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    m[r] = kNegInf;
    lsum[r] = 0.f;
#pragma unroll
    for (int k = 0; k < DK; ++k) acc[r][k] = 0.f;
  }

  const int nblk = (it.n_tok + BS - 1) / BS;
  for (int bi = wave; bi < nblk; bi += 4) {
    const int b = blk[bi];
    const int valid = min(BS, it.n_tok - bi * BS);
    const int64_t tile = layer_tiles + (int64_t)b * p.Hkv + kvh;
    // scores
    float s[MAXR];
#pragma unroll
    for (int r = 0; r < MAXR; ++r) s[r] = 0.f;
    const T* kp = K + (tile * BS + t) * D + part * DPL;
#pragma unroll 2
    for (int c = 0; c < DPL; c += EPV) {
      const u32x4 raw = ld16(kp + c);
      const T* kv = (const T*)&raw;
      float kf[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) kf[e] = to_f32<T>(kv[e]);
#pragma unroll
      for (int r = 0; r < MAXR; ++r) {
        if (r < nr) {
          float a = s[r];
#pragma unroll
          for (int e = 0; e < EPV; ++e) a = fmaf(qs[r][part * DPL + c + e], kf[e], a);
          s[r] = a;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r < nr) {
        float a = s[r];
#pragma unroll
        for (int o = BS; o < 64; o <<= 1) a += __shfl_xor(a, o);
        a *= p.scale_log2;
        if (t >= valid) a = kNegInf;
        float bm = a;
#pragma unroll
        for (int o = 1; o < BS; o <<= 1) bm = fmaxf(bm, __shfl_xor(bm, o));
        const float m_new = fmaxf(m[r], bm);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m[r] - m_use);
        const float pe = fast_exp2(a - m_use);
        lsum[r] = lsum[r] * alpha + (part == 0 ? pe : 0.f);
        m[r] = m_new;
#pragma unroll
        for (int k = 0; k < DK; ++k) acc[r][k] *= alpha;
        if (part == 0) ps[wave][r][t] = pe;
      }
    }
    // make this wave's probabilities visible to all of its lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P.V
#pragma unroll
    for (int k = 0; k < DK; ++k) {
      const int d = lane + 64 * k;
      const T* vp = V + (tile * D + d) * BS;
      float vf[BS];
#pragma unroll
      for (int c = 0; c < BS; c += EPV) {
        const u32x4 raw = ld16(vp + c);
        const T* vv = (const T*)&raw;
#pragma unroll
        for (int e = 0; e < EPV; ++e) vf[c + e] = (c + e < valid) ? to_f32<T>(vv[e]) : 0.f;
      }
#pragma unroll
      for (int r = 0; r < MAXR; ++r) {
        if (r < nr) {
          float a = acc[r][k];
#pragma unroll
          for (int tt = 0; tt < BS; ++tt) a = fmaf(ps[wave][r][tt], vf[tt], a);
          acc[r][k] = a;
        }
      }
    }
    // all lanes have read ps before the next block overwrites it
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    float a = lsum[r];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) a += __shfl_xor(a, o);
    lsum[r] = a;
  }
  // merge the four waves
  if (wave > 0) {
    const int slot = wave - 1;
    for (int r = 0; r < nr; ++r) {
      if (lane == 0) {
        mrg_m[slot][r] = m[r];
        mrg_l[slot][r] = lsum[r];
      }
#pragma unroll
      for (int k = 0; k < DK; ++k) mrg_acc[slot][r][lane + 64 * k] = acc[r][k];
    }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r < nr) {
        for (int slot = 0; slot < 3; ++slot) {
          const float mo = mrg_m[slot][r], lo = mrg_l[slot][r];
          const float M = fmaxf(m[r], mo);
          if (M == kNegInf) continue;
          const float a = fast_exp2(m[r] - M), bb = fast_exp2(mo - M);
          lsum[r] = lsum[r] * a + lo * bb;
#pragma unroll
          for (int k = 0; k < DK; ++k) acc[r][k] = acc[r][k] * a + mrg_acc[slot][r][lane + 64 * k] * bb;
          m[r] = M;
        }
        const int64_t prow = (int64_t)(li * p.Hkv + kvh) * p.P + it.part_row + r;
        if (lane == 0) {
          p.part_ml[2 * prow] = m[r];
          p.part_ml[2 * prow + 1] = lsum[r];
        }
#pragma unroll
        for (int k = 0; k < DK; ++k) p.part_acc[prow * D + lane + 64 * k] = acc[r][k];
      }
    }
  }
}

// ------------------------------------------------------------- combine
//
// Merges each output row's partial states (one per chunk on its path) in
// logical order: M = max m_i, L = sum l_i 2^(m_i - M),
// out = sum acc_i 2^(m_i - M) / L, computed in one online pass. Lane j owns
// d = j*VW .. j*VW + VW-1.
// WPR = 1: a wave per output row, four rows per workgroup (short lists).
// WPR = 4: the four waves of a workgroup split one row's list (long lists:
// split-K over a long context) and merge through LDS.

template <int D, int WPR>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const gbytes_t lb = p.lists_inline ? (gbytes_t)(const uint8_t*)p.lists : (gbytes_t)p.meta_dev;
  const int32_t* comb_ptr = (const int32_t*)(lb + p.off_comb_ptr);
  const int32_t* comb_rows = (const int32_t*)(lb + p.off_comb_rows);
  constexpr int VW = D / 64;
  constexpr int NB = 8;  // partials whose loads are in flight together
  typedef float vec_t __attribute__((ext_vector_type(VW)));
  __shared__ float red_m[4];
  __shared__ float red_l[4];
  __shared__ vec_t red_acc[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n_out = (int64_t)p.n_layers * p.n_branch * p.Hq;
  const int64_t orow = WPR == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
  const bool valid = orow < n_out;
  const int64_t per_layer = (int64_t)p.n_branch * p.Hq;
  const int li = valid ? (int)(orow / per_layer) : 0;
  const int rem = valid ? (int)(orow - li * per_layer) : 0;
  const int b = rem / p.Hq, h = rem - (rem / p.Hq) * p.Hq;
  const int kvh = h / p.G, gq = h - (h / p.G) * p.G;
  const int e0 = valid ? comb_ptr[b] : 0;
  const int e1 = valid ? comb_ptr[b + 1] : 0;
  const int64_t plane = (int64_t)(li * p.Hkv + kvh) * p.P + gq;
  const int sub = WPR == 1 ? 0 : wave;

  // One pass, online: a running maximum M with the sum L and the vector
  // acc scaled by 2^-M, rescaled when M grows. The (m, l, acc) loads of up
  // to NB partials are issued before any of them is used, so a row costs
  // about one memory round trip per NB partials.
  float M = kNegInf, L = 0.f;
  vec_t acc = {};
  for (int e = e0 + sub; e < e1; e += NB * WPR) {
    float mi[NB], li_[NB], mlv[NB];
    vec_t ai[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int ek = e + k * WPR;
      mlv[k] = 0.f;
      ai[k] = vec_t{};
      mi[k] = kNegInf;
      li_[k] = 0.f;
      if (ek < e1) {
        const int64_t row = plane + comb_rows[ek];
        // Long lists (WPR 4) take (m, l) by a vector load, even lanes m and
        // odd lanes l: as a scalar load it would be waited for before the
        // next partial's loads issue (agent combine 7.5 -> 5.6 us). Short
        // lists keep the scalar load, which measured faster for them.
        if constexpr (WPR > 1) {
          mlv[k] = p.part_ml[2 * row + (lane & 1)];
        } else {
          mi[k] = p.part_ml[2 * row];
          li_[k] = p.part_ml[2 * row + 1];
        }
        ai[k] = __builtin_nontemporal_load((const vec_t*)(p.part_acc + row * D + lane * VW));
      }
    }
    if constexpr (WPR > 1) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const bool has = e + k * WPR < e1;
        mi[k] = has ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv[k]), 0)) : kNegInf;
        li_[k] = has ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv[k]), 1)) : 0.f;
      }
    }
    float bm = mi[0];
#pragma unroll
    for (int k = 1; k < NB; ++k) bm = fmaxf(bm, mi[k]);
    const float Mn = fmaxf(M, bm);
    if (Mn != kNegInf) {
      const float a = M == kNegInf ? 0.f : fast_exp2(M - Mn);
      L *= a;
      acc *= a;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float w = mi[k] == kNegInf ? 0.f : fast_exp2(mi[k] - Mn);
        L += li_[k] * w;
        acc += ai[k] * w;
      }
      M = Mn;
    }
  }
  if (WPR > 1) {
    // merge the four waves' states
    if (lane == 0) red_m[wave] = M;
    __syncthreads();
    const float Mt = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
    const float a = (M == kNegInf) ? 0.f : fast_exp2(M - Mt);
    if (lane == 0) red_l[wave] = L * a;
    red_acc[wave][lane] = acc * a;
    __syncthreads();
    if (wave != 0) return;
    L = red_l[0] + red_l[1] + red_l[2] + red_l[3];
    acc = red_acc[0][lane] + red_acc[1][lane] + red_acc[2][lane] + red_acc[3][lane];
  }
  if (!valid) return;
  *(vec_t*)(p.out + orow * D + lane * VW) = acc / L;
}

// ------------------------------------------------------ static scratch
//
// The workspace of pkv_decode_attn_noalloc: plan and partial states of one
// decode, in memory the library never allocates at call time. Host code
// uses only the address hipGetSymbolAddress returns for the current device
// (the array's name in host code is a stand-in, not a device address).

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_pointer(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

struct ArgCopyParams {
  uint8_t* dst;
  int32_t n;
  alignas(16) uint8_t b[kArgCopyBytes];
};

// One workgroup: thread i copies bytes 4i .. 4i + 3 of the payload.
__global__ __launch_bounds__(1024) void arg_copy_kernel(ArgCopyParams p) {
  for (int i = 4 * threadIdx.x; i < p.n; i += 4 * blockDim.x) {
    if (i + 4 <= p.n && ((uintptr_t)(p.dst + i) & 3) == 0) {
      uint32_t v;
      __builtin_memcpy(&v, p.b + i, 4);
      *(uint32_t*)(p.dst + i) = v;
    } else {
      for (int k = i; k < i + 4 && k < p.n; ++k) p.dst[k] = p.b[k];
    }
  }
}

// ------------------------------------------------------------- launchers


hipError_t launch_arg_copy(void* dst, const uint8_t* src, size_t n, hipStream_t stream) {
  ArgCopyParams a;
  for (size_t o = 0; o < n; o += kArgCopyBytes) {
    const size_t m = n - o < (size_t)kArgCopyBytes ? n - o : (size_t)kArgCopyBytes;
    a.dst = (uint8_t*)dst + o;
    a.n = (int32_t)m;
    __builtin_memcpy(a.b, src + o, m);
    arg_copy_kernel<<<dim3(1), dim3(768), 0, stream>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gather(int dtype, const GatherParams& p, hipStream_t stream,
                         const LaunchEvents& ev) {
  if (p.n <= 0) return hipSuccess;
  if (p.n > kGatherSlots) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.n * p.L));
  if (dtype == 0) return launch_kernel(gather_kernel<float>, grid, dim3(256), stream, ev, p);
  return launch_kernel(gather_kernel<uint16_t>, grid, dim3(256), stream, ev, p);
}

hipError_t launch_append(int dtype, const AppendParams& p, hipStream_t stream,
                         const LaunchEvents& ev) {
  const int64_t g64 = (int64_t)p.n_ops * p.L * p.Hkv + (int64_t)p.n_write * p.L;
  if (g64 == 0) return hipSuccess;
  if (g64 > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)g64);
  const dim3 blk(256);
  if (dtype == 0) {
    switch (p.BS) {
      case 16: return launch_kernel(append_kernel<float, 16>, grid, blk, stream, ev, p);
      case 32: return launch_kernel(append_kernel<float, 32>, grid, blk, stream, ev, p);
      case 64: return launch_kernel(append_kernel<float, 64>, grid, blk, stream, ev, p);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.BS) {
    case 16: return launch_kernel(append_kernel<uint16_t, 16>, grid, blk, stream, ev, p);
    case 32: return launch_kernel(append_kernel<uint16_t, 32>, grid, blk, stream, ev, p);
    case 64: return launch_kernel(append_kernel<uint16_t, 64>, grid, blk, stream, ev, p);
    default: return hipErrorInvalidValue;
  }
}

bool append_supported(int BS) { return BS == 16 || BS == 32 || BS == 64; }

bool attn_supported(bool mfma, int dtype, int D, int BS) {
  const bool shape_ok = (D == 64 || D == 128 || D == 256) && (BS == 16 || BS == 32 || BS == 64);
  if (!shape_ok) return false;
  if (mfma) return dtype == 1;
  return dtype == 0 || dtype == 1;
}

namespace {

template <int D, bool LO, bool PF, int RW>
hipError_t launch_mfma_d(int BS, const AttnParams& p, dim3 grid, hipStream_t s, const LaunchEvents& ev) {
  switch (BS) {
    case 16: return launch_kernel(attn_mfma_kernel<D, 16, LO, PF, RW>, grid, dim3(256), s, ev, (const AttnCore&)p, p.meta);
    case 32: return launch_kernel(attn_mfma_kernel<D, 32, LO, PF, RW>, grid, dim3(256), s, ev, (const AttnCore&)p, p.meta);
    default: return launch_kernel(attn_mfma_kernel<D, 64, LO, PF, RW>, grid, dim3(256), s, ev, (const AttnCore&)p, p.meta);
  }
}

template <typename T, int D>
hipError_t launch_valu_d(int BS, const AttnParams& p, dim3 grid, hipStream_t s, const LaunchEvents& ev) {
  switch (BS) {
    case 16: return launch_kernel(attn_valu_kernel<T, D, 16>, grid, dim3(256), s, ev, (const AttnCore&)p, p.meta);
    case 32: return launch_kernel(attn_valu_kernel<T, D, 32>, grid, dim3(256), s, ev, (const AttnCore&)p, p.meta);
    default: return launch_kernel(attn_valu_kernel<T, D, 64>, grid, dim3(256), s, ev, (const AttnCore&)p, p.meta);
  }
}

template <typename T>
hipError_t launch_valu(int D, int BS, const AttnParams& p, dim3 grid, hipStream_t s,
                       const LaunchEvents& ev) {
  if (D == 64) return launch_valu_d<T, 64>(BS, p, grid, s, ev);
  if (D == 128) return launch_valu_d<T, 128>(BS, p, grid, s, ev);
  return launch_valu_d<T, 256>(BS, p, grid, s, ev);
}

}  // namespace

void attn_wide_shape(int D, int* waves, int* row_blocks) {
  // automatic (waves 0 or row_blocks 0): 8 compute waves with two row
  // blocks each up to head_dim 128; at 256 (where two blocks' accumulators
  // would not fit next to three waves per SIMD) 6 waves of one block, which
  // measured faster than 8 (each step reads its K/V from LDS once per wave)
  const bool auto_w = !(*waves == 4 || *waves == 6 || *waves == 8);
  int w = auto_w ? (D == 256 ? 6 : 8) : *waves;
  int r = *row_blocks == 1 || *row_blocks == 2 ? *row_blocks : (D <= 128 ? 2 : 1);
  if (w == 6 || (D == 256 && w == 8)) r = 1;
  *waves = w;
  *row_blocks = r;
}

hipError_t launch_attn_wide(int D, int BS, int waves, int row_blocks, const AttnParams& p,
                            hipStream_t stream, const LaunchEvents& ev) {
  if (!attn_supported(true, 1, D, BS)) return hipErrorInvalidValue;
  int w = waves, r = row_blocks;
  attn_wide_shape(D, &w, &r);
  if (w != waves || r != row_blocks) return hipErrorInvalidValue;
  if (p.n_order == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_order);
#define PKV_WIDE(d, nw, rbw)                                                                    \
  switch (BS) {                                                                                 \
    case 16: return launch_kernel(attn_wide_kernel<d, 16, nw, rbw>, grid, dim3((nw + wide_loaders<d>()) * 64), stream, ev, (const AttnCore&)p, p.meta); \
    case 32: return launch_kernel(attn_wide_kernel<d, 32, nw, rbw>, grid, dim3((nw + wide_loaders<d>()) * 64), stream, ev, (const AttnCore&)p, p.meta); \
    default: return launch_kernel(attn_wide_kernel<d, 64, nw, rbw>, grid, dim3((nw + wide_loaders<d>()) * 64), stream, ev, (const AttnCore&)p, p.meta); \
  }
  if (D == 64) {
    if (w == 8) {
      if (r == 2) PKV_WIDE(64, 8, 2)
      PKV_WIDE(64, 8, 1)
    }
    if (w == 6) PKV_WIDE(64, 6, 1)
    if (r == 2) PKV_WIDE(64, 4, 2)
    PKV_WIDE(64, 4, 1)
  }
  if (D == 128) {
    if (w == 8) {
      if (r == 2) PKV_WIDE(128, 8, 2)
      PKV_WIDE(128, 8, 1)
    }
    if (w == 6) PKV_WIDE(128, 6, 1)
    if (r == 2) PKV_WIDE(128, 4, 2)
    PKV_WIDE(128, 4, 1)
  }
  if (w == 8) PKV_WIDE(256, 8, 1)
  if (w == 6) PKV_WIDE(256, 6, 1)
  if (r == 2) PKV_WIDE(256, 4, 2)
  PKV_WIDE(256, 4, 1)
#undef PKV_WIDE
}

int attn_max_row_blocks_per_wave(int D) { return D <= 128 ? 2 : 1; }

hipError_t launch_attn(bool mfma, bool lo_split, bool prefetch, int row_blocks_per_wave, int dtype,
                       int D, int BS, const AttnParams& p, hipStream_t stream,
                       const LaunchEvents& ev) {
  if (!attn_supported(mfma, dtype, D, BS)) return hipErrorInvalidValue;
  if (p.n_order == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_order);
  if (mfma) {
    if (!lo_split) return hipErrorInvalidValue;  // only the split form is built
    if (row_blocks_per_wave == 2) {
      if (D == 64) return launch_mfma_d<64, true, false, 2>(BS, p, grid, stream, ev);
      if (D == 128) return launch_mfma_d<128, true, false, 2>(BS, p, grid, stream, ev);
      return hipErrorInvalidValue;
    }
    if (row_blocks_per_wave != 1) return hipErrorInvalidValue;
    if (D == 64) return prefetch ? launch_mfma_d<64, true, true, 1>(BS, p, grid, stream, ev)
                                 : launch_mfma_d<64, true, false, 1>(BS, p, grid, stream, ev);
    if (D == 128) return prefetch ? launch_mfma_d<128, true, true, 1>(BS, p, grid, stream, ev)
                                  : launch_mfma_d<128, true, false, 1>(BS, p, grid, stream, ev);
    return prefetch ? launch_mfma_d<256, true, true, 1>(BS, p, grid, stream, ev)
                    : launch_mfma_d<256, true, false, 1>(BS, p, grid, stream, ev);
  }
  if (dtype == 0) return launch_valu<float>(D, BS, p, grid, stream, ev);
  return launch_valu<uint16_t>(D, BS, p, grid, stream, ev);
}

hipError_t launch_combine(int D, int max_entries, const CombineParams& p, hipStream_t stream,
                          const LaunchEvents& ev) {
  const int64_t n_out = (int64_t)p.n_layers * p.n_branch * p.Hq;
  if (n_out == 0) return hipSuccess;
  const bool wide = max_entries >= 8;
  const int64_t g64 = wide ? n_out : (n_out + 3) / 4;
  if (g64 > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)g64);
  if (D == 64) return wide ? launch_kernel(combine_kernel<64, 4>, grid, dim3(256), stream, ev, p)
                           : launch_kernel(combine_kernel<64, 1>, grid, dim3(256), stream, ev, p);
  if (D == 128) return wide ? launch_kernel(combine_kernel<128, 4>, grid, dim3(256), stream, ev, p)
                            : launch_kernel(combine_kernel<128, 1>, grid, dim3(256), stream, ev, p);
  if (D == 256) return wide ? launch_kernel(combine_kernel<256, 4>, grid, dim3(256), stream, ev, p)
                            : launch_kernel(combine_kernel<256, 1>, grid, dim3(256), stream, ev, p);
  return hipErrorInvalidValue;
}

}  // namespace pkv
