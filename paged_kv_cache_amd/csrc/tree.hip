// Tree attention (decode) for gfx950: one workgroup per (tree item, layer,
// KV head) reads every chunk the item's rows hold -- a tree's shared root
// and each of its edges -- exactly once, applies it to the rows that hold it
// and writes the final output rows. For a deep tree (an MCTS tree: a root
// held by all leaves, then edges held by fewer and fewer) the shared root is
// a dense contraction over all rows and the edges are memory traffic; no
// partial state is written and no second launch re-reads the edges per
// leaf. (On the MCTS batch it measures slower than the wide root launch
// followed by the narrow leaf launch: each step is one barrier-synchronised
// walk of all eight waves, and on an edge only the waves holding its rows
// work while the rest wait.)
//
// Shape: 8 waves, two per SIMD, each owning 32 rows (two 16-row blocks), so
// every K/V operand read from LDS feeds two matrix products. Each wave also
// moves its eighth of every 32-token step of K/V from global memory into
// LDS (global_load_lds_dwordx4, operand order, as the wide kernel's loaders
// do) into a ring of NS separate LDS arrays. Two waves per SIMD leave each
// up to 256 registers (VGPRs and AGPRs).
//
// Per step and wave: the next step's Q.K^T for both blocks from one read of
// its K sections (issued first), then this step's row maxima, per block the
// probabilities (bf16 hi + lo, as in the other kernels) and its P.V
// products from one read of the V sections, the second block's
// probabilities placed between the first block's products.
//
// Chunks whose row mask leaves some rows out (the edges) skip the row blocks
// with no row in the mask and give masked rows -inf scores. Odd planes walk
// the chunk list backwards.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "kernel_common.h"
#include "kernels.hpp"

namespace pkv {

namespace {

// A position in an item's step sequence: chunk i of the walk (chunk ci of
// the list), step s of that chunk.
struct Cursor {
  int i, ci, s, nst, ntok, blk;
};

}  // namespace

// One 16-byte-per-lane load of global memory into LDS (the lane's 16 bytes
// land at lds + 16 * lane), written out so that the compiler does not track
// it: the load writes no register, and the kernel orders every LDS read of
// the data after its own s_waitcnt and barrier. (Through the builtin, the
// compiler would wait for every load in flight before each LDS read of the
// same wave, since it cannot tell the ring's stages apart.)
// m0 (which holds the LDS address) is saved and restored around it: the
// compiler treats m0 as reserved and may not honour a clobber of it.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// P.V for one 16-row block is acc[j] += V^T[16j .. 16j + 15][32 tokens] P^T
// with P = hi + lo (two products per d block) and the accumulators held in
// AGPRs, written as asm (pv_step_if below) so that they stay there: given
// the builtin, the compiler moves the accumulators into VGPRs, and the
// blocks' accumulators do not fit beside the rest. The two products into
// one accumulator run back to back (same shape, exact overlap: no wait). An
// accumulator is read back by other code only after settle() below.

// Q.K^T for a wave's two 16-row blocks: per block the two 16-token score
// tiles of a 32-token step, s[r][tau] = K[tau] Q_r^T (rows of the tile are
// tokens, columns the block's rows), with the queries held in AGPRs (matrix
// products read their B operand from there). The four chains (block, tile)
// are interleaved so that no product waits on the one just before it.
// on0 / on1 (wave-uniform) skip a block with no row in the step's mask; its
// scores are left unspecified (every one of them is masked afterwards).
// The statement always runs (a C++ branch around it would let the compiler
// copy fresh results at the join, with no wait for the products); the
// scores are read by vector instructions only a whole step later.
template <int KS>
__device__ __forceinline__ void qk_pair(f32x4 (&s)[2][2], const u32x4 (&k)[2 * KS],
                                        const bf16x8 (&q0)[KS], const bf16x8 (&q1)[KS],
                                        uint32_t on0, uint32_t on1);
template <>
__device__ __forceinline__ void qk_pair<4>(f32x4 (&s)[2][2], const u32x4 (&k)[8],
                                           const bf16x8 (&q0)[4], const bf16x8 (&q1)[4],
                                           uint32_t on0, uint32_t on1) {
  asm("s_cmp_eq_u32 %20, 0\n\t"
      "s_cbranch_scc1 3f\n\t"
      "s_cmp_eq_u32 %21, 0\n\t"
      "s_cbranch_scc1 2f\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %12, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %8, %12, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %4, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %8, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %13, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %9, %13, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %5, %17, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %9, %17, %3\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %14, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %10, %14, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %6, %18, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %10, %18, %3\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %7, %15, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %11, %15, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %7, %19, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %11, %19, %3\n\t"
      "s_branch 4f\n"
      "2:\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %12, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %8, %12, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %13, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %9, %13, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %14, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %10, %14, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %7, %15, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %11, %15, %1\n\t"
      "s_branch 4f\n"
      "3:\n\t"
      "s_cmp_eq_u32 %21, 0\n\t"
      "s_cbranch_scc1 4f\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %4, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %8, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %5, %17, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %9, %17, %3\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %6, %18, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %10, %18, %3\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %7, %19, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %11, %19, %3\n"
      "4:"
      : "=&v"(s[0][0]), "=&v"(s[0][1]), "=&v"(s[1][0]), "=&v"(s[1][1])
      : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]),
        "a"(q0[0]), "a"(q0[1]), "a"(q0[2]), "a"(q0[3]), "a"(q1[0]), "a"(q1[1]), "a"(q1[2]),
        "a"(q1[3]), "s"(__builtin_amdgcn_readfirstlane(on0)),
        "s"(__builtin_amdgcn_readfirstlane(on1))
      : "scc");
}
template <>
__device__ __forceinline__ void qk_pair<2>(f32x4 (&s)[2][2], const u32x4 (&k)[4],
                                           const bf16x8 (&q0)[2], const bf16x8 (&q1)[2],
                                           uint32_t on0, uint32_t on1) {
  asm("s_cmp_eq_u32 %12, 0\n\t"
      "s_cbranch_scc1 3f\n\t"
      "s_cmp_eq_u32 %13, 0\n\t"
      "s_cbranch_scc1 2f\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %8, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %8, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %4, %10, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %6, %10, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %9, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %7, %9, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %5, %11, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %7, %11, %3\n\t"
      "s_branch 4f\n"
      "2:\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %8, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %8, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %9, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %7, %9, %1\n\t"
      "s_branch 4f\n"
      "3:\n\t"
      "s_cmp_eq_u32 %13, 0\n\t"
      "s_cbranch_scc1 4f\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %4, %10, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %6, %10, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %5, %11, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %7, %11, %3\n"
      "4:"
      : "=&v"(s[0][0]), "=&v"(s[0][1]), "=&v"(s[1][0]), "=&v"(s[1][1])
      : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "a"(q0[0]), "a"(q0[1]), "a"(q1[0]),
        "a"(q1[1]), "s"(__builtin_amdgcn_readfirstlane(on0)),
        "s"(__builtin_amdgcn_readfirstlane(on1))
      : "scc");
}


// A block's queries (KS 16-byte pieces per lane, 64 bytes apart) loaded
// straight into AGPRs, the load waited for in the same statement: defined
// in AGPRs, they stay there (loaded into VGPRs, the compiler would copy them
// into AGPRs before every product).
template <int KS>
__device__ __forceinline__ void load_q(bf16x8 (&q)[KS], const void* src);
template <>
__device__ __forceinline__ void load_q<4>(bf16x8 (&q)[4], const void* src) {
  asm volatile(
      "global_load_dwordx4 %0, %4, off\n\t"
      "global_load_dwordx4 %1, %4, off offset:64\n\t"
      "global_load_dwordx4 %2, %4, off offset:128\n\t"
      "global_load_dwordx4 %3, %4, off offset:192\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&a"(q[0]), "=&a"(q[1]), "=&a"(q[2]), "=&a"(q[3])
      : "v"(src)
      : "memory");
}
template <>
__device__ __forceinline__ void load_q<2>(bf16x8 (&q)[2], const void* src) {
  asm volatile(
      "global_load_dwordx4 %0, %2, off\n\t"
      "global_load_dwordx4 %1, %2, off offset:64\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&a"(q[0]), "=&a"(q[1])
      : "v"(src)
      : "memory");
}

// An accumulator set to zero by a matrix product (0 x 0 + 0), so that it
// is defined in AGPRs: zeroed by ordinary code it would be defined in VGPRs,
// and the compiler would carry it there, copying it into AGPRs and back
// around every product. Volatile: the statements of all accumulators have
// the same input, and merged into one, the compiler would copy its result
// into the others with no wait for the product (it does not know the
// statement holds one). The caller settles the accumulators before any
// other code reads them.
__device__ __forceinline__ void zero_acc(f32x4& acc, const u32x4& z) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}

// One d block of a row block's P.V, hi then lo, for a block that may have
// no row in the chunk's mask (on == 0: skip both products). The skip is a
// branch inside the statement, so that for the compiler the accumulator is
// always rewritten by it: a branch around it in C++ would make the compiler
// copy every accumulator at the join. s_nop 1 gives the two wait states a
// vector write of an operand needs before a product reads it.
__device__ __forceinline__ void pv_step_if(f32x4& acc, const u32x4& v, bf16x8 phi, bf16x8 plo,
                                           uint32_t on) {
  asm("s_cmp_eq_u32 %4, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "s_nop 1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %1, %3, %0\n"
      "1:"
      : "+a"(acc)
      : "v"(v), "v"(phi), "v"(plo), "s"(__builtin_amdgcn_readfirstlane(on))
      : "scc");
}

// The probabilities of one row block's eight scores per lane (as probs8:
// p = 2^(s c - m), bf16 hi and its rounding residual lo), computed in eight
// slices so that they can be interleaved with another block's products:
// even slices take two exponentials, odd slices convert that pair.
struct Probs {
  float p[8];
  float psum;
  bf16x8 phi, plo;
};
template <int K>
__device__ __forceinline__ void probs_slice(Probs& q, const float (&sc)[8], float c, float m) {
  constexpr int e = 2 * (K >> 1);
  if constexpr ((K & 1) == 0) {
    q.p[e] = fast_exp2(__builtin_fmaf(sc[e], c, -m));
    q.p[e + 1] = fast_exp2(__builtin_fmaf(sc[e + 1], c, -m));
    q.psum += q.p[e] + q.p[e + 1];
  } else {
    const bf16x2 h = __builtin_convertvector((f32x2){q.p[e], q.p[e + 1]}, bf16x2);
    q.phi[e] = h[0];
    q.phi[e + 1] = h[1];
    const f32x2 hf = __builtin_convertvector(h, f32x2);
    const bf16x2 l = __builtin_convertvector((f32x2){q.p[e] - hf[0], q.p[e + 1] - hf[1]}, bf16x2);
    q.plo[e] = l[0];
    q.plo[e + 1] = l[1];
  }
}
template <int K0, int K1>
__device__ __forceinline__ void probs_slices(Probs& q, const float (&sc)[8], float c, float m) {
  if constexpr (K0 < K1) {
    probs_slice<K0>(q, sc, c, m);
    probs_slices<K0 + 1, K1>(q, sc, c, m);
  }
}

// Block r's P.V products (DB statements), statement j followed by slices
// [8j / DB, 8(j + 1) / DB) of the next block's probabilities (NEXT), each
// pair fenced so that the scheduler keeps this interleaving.
template <int J, int DB, bool NEXT>
__device__ __forceinline__ void pv_interleaved(f32x4 (&acc)[DB], const u32x4 (&v)[DB],
                                               const Probs& cur, Probs& nxt,
                                               const float (&sc)[8], float c, float m,
                                               uint32_t on) {
  if constexpr (J < DB) {
    pv_step_if(acc[J], v[J], cur.phi, cur.plo, on);
    if constexpr (NEXT) probs_slices<8 * J / DB, 8 * (J + 1) / DB>(nxt, sc, c, m);
    __builtin_amdgcn_sched_barrier(0);
    pv_interleaved<J + 1, DB, NEXT>(acc, v, cur, nxt, sc, c, m, on);
  }
}

// Waits out the products still writing a block's accumulators (an XDL
// product's result is readable by other instructions some 19 wait states
// after it issues at the longest) before the compiler's own code reads or
// rewrites them.
template <int DB>
__device__ __forceinline__ void settle(f32x4 (&acc)[DB]) {
  if constexpr (DB == 8)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]),
                   "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
}

// NEG: the softmax scale is negative; the scores are negated before they
// are masked (the scale's magnitude is folded into the exponent as
// elsewhere).
//
// The walk is software-pipelined by one step: step t + 1 is made visible
// (its loads waited for, then a barrier) before step t is finished, so that
// each wave issues step t + 1's score products first and computes step t's
// maxima, probabilities and P.V while they run. Two ring stages are in use
// at a time (step t's V, step t + 1's K), so NS - 3 steps of loads stay in
// flight behind them.
template <int D, int BS, int NS, bool NEG>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_tree_kernel(AttnCore p, PlanBytes plan_bytes) {
  constexpr int KS = D / 32;           // 32-wide k steps of Q.K
  constexpr int DB = D / 16;           // 16-wide d blocks of P.V
  constexpr int NSEC = 2 * KS + DB;    // 1 KiB operand sections per step
  constexpr int NW = 8;                // waves (each loads and computes)
  constexpr int RBW = 2;               // 16-row blocks per wave
  constexpr int RPW = 16 * RBW;        // rows per wave
  constexpr int NT = 64 * NW;          // threads
  constexpr int SPL = NSEC / NW;       // sections each wave loads per step
  static_assert(NW * RPW == kTreeRows && 64 % RPW == 0 && RBW == 2, "rows per wave");
  static_assert(NSEC % NW == 0, "sections per wave");
  static_assert(NS >= 4 && NS <= 6, "ring stages");
  static_assert((NS - 1) * SPL < 64, "loads in flight per wave");
  static_assert(BS == 16 || BS == 32 || BS == 64, "block size");
  __shared__ u32x4 ring[NS][NSEC * 64];
  __shared__ int redo_s;

  const PlanArrays sp = plan_arrays(p, plan_bytes);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int planes = p.n_layers * p.Hkv;
  const int item_idx = blockIdx.x / planes;
  const int plane = blockIdx.x - item_idx * planes;
  const int li = plane / p.Hkv;
  const int kvh = plane - li * p.Hkv;
  const int layer = p.layer0 + li;
  const TreeItem ti = sp.titems[item_idx];
  // The item's block ids and chunk records are read with scalar loads
  // (constant address space: wave-uniform, read-only): in LDS they would
  // queue behind the operand traffic, on every wave's critical path.
  typedef const __attribute__((address_space(4))) int32_t* CBlk;
  typedef const __attribute__((address_space(4))) TreeChunk* CChunk;
  const CBlk blk_c = (CBlk)(sp.blk + ti.blk_off);
  const CChunk ch_c = (CChunk)(sp.tchunks + ti.chunk_off);
  const bool rev = plane & 1;
  const int n_chunks = ti.n_chunks;
  const int total = ti.n_steps;

  auto enter = [&](Cursor& c, int i) __attribute__((always_inline)) {
    c.i = i;
    c.ci = rev ? n_chunks - 1 - i : i;
    c.s = 0;
    c.ntok = ch_c[c.ci].n_tok;
    c.nst = ch_c[c.ci].n_steps;
    c.blk = ch_c[c.ci].blk_off;
  };
  // next step; at the last step of the walk the cursor stays (loads issued
  // past the end re-read that step, in bounds, into a stage never read)
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    if (c.s + 1 < c.nst) {
      ++c.s;
    } else if (c.i + 1 < n_chunks) {
      enter(c, c.i + 1);
    }
  };

  // ------------------------------------------------------------- loads
  const int koff0 = 8 * (n >> 2) + (n & 3);
  const int voff = 8 * g;
  // this plane's (layer, KV head) tile of block 0; block b's is b * tile_step further
  const int64_t tile_step = (int64_t)p.Hkv * BS * D;
  const uint16_t* Kp = (const uint16_t*)p.k_arena + ((int64_t)layer * p.num_blocks * p.Hkv + kvh) * BS * D;
  const uint16_t* Vp = (const uint16_t*)p.v_arena + ((int64_t)layer * p.num_blocks * p.Hkv + kvh) * BS * D;
  const uint32_t ring_base = (uint32_t)(uintptr_t)&ring[0][0];
  // The block ids of the cursor's step (tokens tb .. tb + 15 and
  // tb + 16 .. tb + 31), loaded a step before they are used.
  struct Ids {
    int a, b;
  };
  auto ids_of = [&](const Cursor& c) __attribute__((always_inline)) {
    const int tb = 32 * c.s;
    Ids r;
    r.a = blk_c[c.blk + tb / BS];
    r.b = blk_c[c.blk + (tb + 16) / BS];
    return r;
  };
  // Sections wave + NW * k of the cursor's step into stage st: sections
  // below 2KS are K, the rest V. The block ids are wave-uniform (scalar
  // offsets); only the lane's place in the tile is per lane.
  auto issue = [&](const Cursor& c, const Ids& id, int st) __attribute__((always_inline)) {
    const int tb = 32 * c.s;
    const int64_t oA = (int64_t)id.a * tile_step, oB = (int64_t)id.b * tile_step;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int sect = wave + NW * k;
      const uint16_t* src;
      if (sect < 2 * KS) {
        const int tau = sect / KS, ks = sect - (sect / KS) * KS;
        const int off = koff0 + 4 * tau;
        src = Kp + ((BS == 16 && off >= 16) ? oB : oA) + ((tb + off) % BS) * D + 32 * ks + 8 * g;
      } else {
        const int j = sect - 2 * KS;
        src = Vp + ((BS == 16 && voff >= 16) ? oB : oA) + (16 * j + n) * BS + (tb + voff) % BS;
      }
      dma16(src, ring_base + (uint32_t)((st * NSEC + sect) * 1024));
    }
  };
  // In a chunk's last, ragged step the V slots past its end may hold
  // anything (even NaN): each wave zeroes them in the V sections it loaded,
  // after they land and before the barrier, so that 0 * V stays 0.
  auto zero_tail = [&](const Cursor& c, int st) __attribute__((always_inline)) {
    const int tv = 32 * c.s + voff;
    u32x4 keep;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = (tv + 2 * w < c.ntok) ? 0x0000ffffu : 0u;
      const uint32_t hi = (tv + 2 * w + 1 < c.ntok) ? 0xffff0000u : 0u;
      keep[w] = lo | hi;
    }
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int sect = wave + NW * k;
      if (sect >= 2 * KS) ring[st][sect * 64 + lane] &= keep;
    }
    // the writes land before the barrier that publishes them (s_barrier
    // alone does not wait for them): lgkmcnt(0), no wait on the others
    __builtin_amdgcn_s_waitcnt(0xC07F);
  };

  // ----------------------------------------------------------- queries
  // (rows past the item's last read the first holder's query; their
  // results are never written)
  bf16x8 qv[RBW][KS];
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    int row = RPW * wave + 16 * r + n;
    if (row >= ti.n_rows) row = 0;
    const int hold = row / p.G;
    const int gq = row - hold * p.G;
    const int branch = sp.holders[ti.hold_off + hold];
    const uint16_t* qp = (const uint16_t*)p.q +
                         (((int64_t)li * p.n_branch + branch) * p.Hq + kvh * p.G + gq) * D + 8 * g;
    load_q<KS>(qv[r], qp);
  }

  f32x4 acc[RBW][DB];
  // m_ref: each row's reference for its probabilities, fixed once set (the
  // first finite score maximum in the first pass, the row's true maximum in
  // a second); m_max: the row's running maximum; l_run: its running sum.
  float m_ref[RBW], m_max[RBW], l_run[RBW];
  const float cs = p.abs_scale_log2;

  // ------------------------------------------------------------- steps
  // A step as one wave sees it: m holds the wave's rows in the chunk's
  // mask (row 16 r + n at bit 16 r + n), tb the step's first token in the
  // chunk, st its ring stage; full: every row in, no token past the end.
  struct Step {
    uint32_t m;
    int tb, ntok, st;
    bool full;
  };
  auto step_of = [&](const Cursor& c, int st) __attribute__((always_inline)) {
    Step s;
    const uint64_t rows = ch_c[c.ci].rows[(RPW * wave) >> 6];
    s.m = (uint32_t)(rows >> ((RPW * wave) & 63));
    s.tb = 32 * c.s;
    s.ntok = c.ntok;
    s.st = st;
    s.full = s.m == ~0u && s.tb + 32 <= c.ntok;
    return s;
  };
  auto block_on = [&](const Step& s, int r) __attribute__((always_inline)) {
    return (s.full || ((s.m >> (16 * r)) & 0xFFFFu) != 0) ? 1u : 0u;
  };
  // Q.K^T of a step for both blocks, into sc (issued; read a step later).
  // A wave with no row in the step reads no K (the products are skipped).
  auto scores = [&](const Step& s, f32x4 (&sc)[RBW][2]) __attribute__((always_inline)) {
    u32x4 kreg[2 * KS];
    if (s.m != 0) {
      const u32x4* buf = ring[s.st];
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) kreg[i] = buf[i * 64 + lane];
    }
    const uint32_t on0 = s.m != 0 ? block_on(s, 0) : 0u;
    const uint32_t on1 = s.m != 0 ? block_on(s, 1) : 0u;
    qk_pair<KS>(sc, kreg, qv[0], qv[1], on0, on1);
  };
  // block r's scores to masked values x and their reference mu; the row's
  // running maximum and (first pass) its first finite maximum updated
  auto row_max = [&](const Step& s, const f32x4 (&sc)[2], int r, float (&x)[8], float& mu,
                     bool first_pass) __attribute__((always_inline)) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * tau + i] = sc[tau][i];
    if (NEG) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = -x[e];
    }
    // (after the negation: a masked score stays -inf)
    if (!s.full) {
      const int valid = ((s.m >> (16 * r + n)) & 1u) ? s.ntok - (s.tb + voff) : 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = e < valid ? x[e] : kNegInf;
    }
    const float mx = max_xor32(max_xor16(rmax8(x))) * cs;
    m_max[r] = rmax(m_max[r], mx);
    // the first finite maximum becomes the reference (nothing has been
    // accumulated yet, so nothing is rescaled)
    if (first_pass && m_ref[r] == kNegInf) m_ref[r] = mx;
    mu = (m_ref[r] == kNegInf) ? 0.f : m_ref[r];
  };

  // One iteration: make step t + 1 visible and load step t + NS - 1 into
  // the stage step t - 1 used; issue step t + 1's score products; finish
  // step t from its scores (cur): maxima, probabilities, P.V. nxt receives
  // step t + 1's scores.
  constexpr int kWait = (NS - 3) * SPL;
  constexpr int kWaitVm = 0x0F70 | (kWait & 0xF) | ((kWait >> 4) << 14);
  Cursor ld, cq;
  Step cur_s, nxt_s;  // steps t and t + 1 (nxt_s read a step ahead)
  Ids ld_ids;         // block ids of ld's step, read a step ahead
  int st_next = 0, st_free = 0;
  auto iter = [&](int t, f32x4 (&cur)[RBW][2], f32x4 (&nxt)[RBW][2], bool first_pass)
      __attribute__((always_inline)) {
    const bool more = t + 1 < total;
    __builtin_amdgcn_s_waitcnt(kWaitVm);
    if (more && cq.s == cq.nst - 1 && (cq.ntok & 31) != 0) zero_tail(cq, st_next);
    __builtin_amdgcn_s_barrier();
    issue(ld, ld_ids, st_free);
    advance(ld);
    ld_ids = ids_of(ld);
    Step nx_s = nxt_s;
    if (!more) nx_s.m = 0u;
    const Step s = cur_s;
    float x[RBW][8], mu[RBW];
    u32x4 vreg[DB];
    uint32_t act[RBW];
    if (s.m != 0) {
#pragma unroll
      for (int r = 0; r < RBW; ++r) {
        act[r] = block_on(s, r);
        row_max(s, cur[r], r, x[r], mu[r], first_pass);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    scores(nx_s, nxt);
    __builtin_amdgcn_sched_barrier(0);
    if (s.m != 0) {
      // (the V operands after the K ones are dead; their reads overlap
      // block 0's probabilities)
      const u32x4* buf = ring[s.st];
#pragma unroll
      for (int j = 0; j < DB; ++j) vreg[j] = buf[(2 * KS + j) * 64 + lane];
      // block 0's probabilities, then its products, each followed by a
      // slice of block 1's probabilities, then block 1's products
      Probs p0, p1;
      p0.psum = 0.f;
      p1.psum = 0.f;
      probs_slices<0, 8>(p0, x[0], cs, mu[0]);
      __builtin_amdgcn_sched_barrier(0);
      pv_interleaved<0, DB, true>(acc[0], vreg, p0, p1, x[1], cs, mu[1], act[0]);
      pv_interleaved<0, DB, false>(acc[1], vreg, p1, p1, x[1], cs, mu[1], act[1]);
      l_run[0] += p0.psum;
      l_run[1] += p1.psum;
    }
    advance(cq);
    st_free = s.st;
    cur_s = nx_s;
    st_next = st_next + 1 == NS ? 0 : st_next + 1;
    nxt_s = step_of(cq, st_next);
  };

#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    m_ref[r] = kNegInf;
    m_max[r] = kNegInf;
  }
  f32x4 scA[RBW][2], scB[RBW][2];
  for (int pass = 0; pass < 2; ++pass) {
    // (a second pass: the first one's output stores are still counted in
    // vmcnt; let them finish, so that the counted waits below see loads only)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
#pragma unroll
      for (int j = 0; j < DB; ++j) zero_acc(acc[r][j], zero);
      l_run[r] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < RBW; ++r) settle<DB>(acc[r]);
    // steps 0 .. NS - 2 into stages 0 .. NS - 2; step 0 visible; its scores
    enter(ld, 0);
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
      issue(ld, ids_of(ld), k);
      advance(ld);
    }
    ld_ids = ids_of(ld);
    enter(cq, 0);
    {
      constexpr int kW0 = (NS - 2) * SPL;
      __builtin_amdgcn_s_waitcnt(0x0F70 | (kW0 & 0xF) | ((kW0 >> 4) << 14));
    }
    if (cq.s == cq.nst - 1 && (cq.ntok & 31) != 0) zero_tail(cq, 0);
    __builtin_amdgcn_s_barrier();
    cur_s = step_of(cq, 0);
    scores(cur_s, scA);
    advance(cq);
    st_next = 1;
    st_free = NS - 1;
    nxt_s = step_of(cq, st_next);
    for (int t = 0; t < total; t += 2) {
      iter(t, scA, scB, pass == 0);
      if (t + 1 < total) iter(t + 1, scB, scA, pass == 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the walk

    // ---------------------------------------------------------- output
    bool bad = false;
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
      settle<DB>(acc[r]);
      const float l_tot = sum_xor32(sum_xor16(l_run[r]));
      const int row = RPW * wave + 16 * r + n;
      if (row >= ti.n_rows) continue;
      const int hold = row / p.G;
      const int gq = row - hold * p.G;
      const int branch = sp.holders[ti.hold_off + hold];
      float* orow = p.out + (((int64_t)li * p.n_branch + branch) * p.Hq + kvh * p.G + gq) * D;
      const float inv = 1.f / l_tot;
      bad = bad || !__builtin_isfinite(inv) || !__builtin_isfinite(l_tot);
#pragma unroll
      for (int j = 0; j < DB; ++j) {
        const f32x4 o = acc[r][j] * inv;
        bad = bad || !__builtin_isfinite(o[0]) || !__builtin_isfinite(o[1]) ||
              !__builtin_isfinite(o[2]) || !__builtin_isfinite(o[3]);
        *(f32x4*)(orow + 16 * j + 4 * g) = o;
      }
    }
    // A row whose first maximum lay far below its true one can overflow
    // (probabilities of up to 2^(m_max - m_ref)): then the whole workgroup
    // walks again with every row's true maximum as its reference, where no
    // probability exceeds 1, and overwrites its outputs.
    if (pass == 1) break;
    __syncthreads();
    if (threadIdx.x == 0) redo_s = 0;
    __syncthreads();
    if (__any(bad) && lane == 0) redo_s = 1;
    __syncthreads();
    if (!redo_s) break;
#pragma unroll
    for (int r = 0; r < RBW; ++r) m_ref[r] = m_max[r];
  }
}

// ------------------------------------------------------------- launcher

bool tree_supported(int D, int BS) {
  return (D == 64 || D == 128) && (BS == 16 || BS == 32 || BS == 64);
}

hipError_t launch_attn_tree(int D, int BS, int stages, const AttnParams& p, int n_wg,
                            hipStream_t stream, const LaunchEvents& ev) {
  if (!tree_supported(D, BS) || stages < 4 || stages > 6) return hipErrorInvalidValue;
  if (n_wg <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_wg), block(512);
  const bool neg = p.q_flip != 0;  // a negative softmax scale
#define PKV_TREE_NS(d, bs, ns)                                                                   \
  return neg ? launch_kernel(attn_tree_kernel<d, bs, ns, true>, grid, block, stream, ev,         \
                             (const AttnCore&)p, p.meta)                                         \
             : launch_kernel(attn_tree_kernel<d, bs, ns, false>, grid, block, stream, ev,        \
                             (const AttnCore&)p, p.meta);
#define PKV_TREE(d, bs)               \
  if (D == d && BS == bs) {           \
    if (stages == 4) {                \
      PKV_TREE_NS(d, bs, 4)           \
    } else if (stages == 5) {         \
      PKV_TREE_NS(d, bs, 5)           \
    } else {                          \
      PKV_TREE_NS(d, bs, 6)           \
    }                                 \
  }
  PKV_TREE(64, 16)
  PKV_TREE(64, 32)
  PKV_TREE(64, 64)
  PKV_TREE(128, 16)
  PKV_TREE(128, 32)
  PKV_TREE(128, 64)
#undef PKV_TREE
#undef PKV_TREE_NS
  return hipErrorInvalidValue;
}

}  // namespace pkv
