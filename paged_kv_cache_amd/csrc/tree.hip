// Tree attention (decode) for gfx950: one workgroup per (tree item, layer,
// KV head) reads every chunk the item's rows hold -- a tree's shared root
// and each of its edges -- exactly once, applies it to the rows that hold it
// and writes the final output rows. For a deep tree (an MCTS tree: a root
// held by all leaves, then edges held by fewer and fewer) the shared root is
// a dense contraction over all rows and the edges are memory traffic; in one
// workgroup per plane the two overlap across the chip, no partial state is
// written and no second launch re-reads the edges per leaf.
//
// Shape: 4 waves, one per SIMD, each owning 64 rows (four 16-row blocks), so
// every K/V operand read from LDS feeds four matrix products. Each wave also
// moves its quarter of every 32-token step of K/V from global memory into
// LDS (global_load_lds_dwordx4, operand order, as the wide kernel's loaders
// do), keeping NS - 1 steps in flight in a ring of NS separate LDS arrays.
// One wave per SIMD leaves each wave up to 512 registers (VGPRs and AGPRs),
// room for the four blocks' accumulators next to the softmax and operands.
//
// Per step and wave (all four blocks active): Q.K^T for the four blocks from
// one read of the K sections, the four row maxima and one wave vote for the
// (rare) rescale, then per block the probabilities (bf16 hi + lo, as in the
// other kernels) and its P.V products from one read of the V sections; the
// blocks' softmax and products are independent, so the scheduler overlaps
// one block's vector work with another block's matrix products.
//
// Chunks whose row mask leaves some rows out (the edges) skip the row blocks
// with no row in the mask and give masked rows -inf scores. Odd planes walk
// the chunk list backwards, so at any moment about half the workgroups are
// in a compute-heavy stretch (the root) and half in a memory-heavy one.
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

// P.V for one 16-row block: acc[j] += V^T[16j .. 16j + 15][32 tokens] P^T,
// P = hi + lo (two products per d block), with the accumulators held in
// AGPRs: written as asm so that they stay there (given the builtin, the
// compiler moves accumulators that the rare rescale multiplies into VGPRs,
// and four blocks of them do not fit beside the rest). One statement per d
// block, so that the scheduler can place the vector work of another block
// between them. s_nop 1 gives the two wait states a VALU write of an
// operand needs before a matrix product reads it; the two products into one
// accumulator run back to back (same shape, exact overlap: no wait). An
// accumulator is read back by other code only after settle() below.
__device__ __forceinline__ void pv_step(f32x4& acc, const u32x4& v, bf16x8 phi, bf16x8 plo) {
  asm("s_nop 1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %1, %3, %0"
      : "+a"(acc)
      : "v"(v), "v"(phi), "v"(plo));
}

// Q.K^T for one 16-row block: the two 16-token score tiles of a 32-token
// step, S^T[tau] = sum_ks K[tau][ks] Q^T[ks], with the block's queries held
// in AGPRs (matrix products read their B operand from there), which keeps
// 64 VGPRs free for the rest. on == 0 skips the block (its scores are left
// unspecified; every score of such a block is masked afterwards) and waits
// out the products of the block before, whose scores are read next. The
// scores are read by vector instructions only after another block's
// statement or after settle_v(), which waits out the writes.
template <int KS>
__device__ __forceinline__ void qk_block(f32x4& s0, f32x4& s1, const u32x4 (&k)[2 * KS],
                                         const bf16x8 (&q)[KS], uint32_t on);
template <>
__device__ __forceinline__ void qk_block<4>(f32x4& s0, f32x4& s1, const u32x4 (&k)[8],
                                            const bf16x8 (&q)[4], uint32_t on) {
  asm("s_cmp_eq_u32 %14, 0\n\t"
      "s_cbranch_scc0 2f\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
      "s_branch 1f\n"
      "2:\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %10, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %10, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %11, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %7, %11, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %12, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %8, %12, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %13, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %9, %13, %1\n"
      "1:"
      : "=&v"(s0), "=&v"(s1)
      : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]),
        "a"(q[0]), "a"(q[1]), "a"(q[2]), "a"(q[3]), "s"(__builtin_amdgcn_readfirstlane(on))
      : "scc");
}
template <>
__device__ __forceinline__ void qk_block<2>(f32x4& s0, f32x4& s1, const u32x4 (&k)[4],
                                            const bf16x8 (&q)[2], uint32_t on) {
  asm("s_cmp_eq_u32 %8, 0\n\t"
      "s_cbranch_scc0 2f\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
      "s_branch 1f\n"
      "2:\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %6, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %6, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %7, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %7, %1\n"
      "1:"
      : "=&v"(s0), "=&v"(s1)
      : "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "a"(q[0]), "a"(q[1]), "s"(__builtin_amdgcn_readfirstlane(on))
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
// around every product.
__device__ __forceinline__ void zero_acc(f32x4& acc, const u32x4& z) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}

__device__ __forceinline__ void settle_v(f32x4& s0, f32x4& s1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0), "+v"(s1));
}

// pv_step for a block that may have no row in the chunk's mask (on == 0:
// skip both products). The skip is a branch inside the statement, so that
// for the compiler the accumulator is always rewritten by it: a branch
// around it in C++ would make the compiler copy every accumulator at the
// join.
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

// acc *= alpha (per lane) in place, in the accumulator's own AGPRs; the
// products still writing it are waited out first (an XDL result is read by
// other instructions some 19 wait states after issue at the longest).
__device__ __forceinline__ void scale_acc(f32x4& acc, float alpha) {
  float e0 = acc[0], e1 = acc[1], e2 = acc[2], e3 = acc[3];
  float t;
  asm volatile(
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
      "v_accvgpr_read_b32 %4, %0\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %0, %4\n\t"
      "v_accvgpr_read_b32 %4, %1\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %1, %4\n\t"
      "v_accvgpr_read_b32 %4, %2\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %2, %4\n\t"
      "v_accvgpr_read_b32 %4, %3\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %3, %4"
      : "+a"(e0), "+a"(e1), "+a"(e2), "+a"(e3), "=&v"(t)
      : "v"(alpha));
  acc = f32x4{e0, e1, e2, e3};
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

// NEG: the softmax scale is negative; the scores are negated as they are
// masked (the scale's magnitude is folded into the exponent as elsewhere).
template <int D, int BS, int NS, bool NEG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_tree_kernel(AttnCore p, PlanBytes plan_bytes) {
  constexpr int KS = D / 32;           // 32-wide k steps of Q.K
  constexpr int DB = D / 16;           // 16-wide d blocks of P.V
  constexpr int NSEC = 2 * KS + DB;    // 1 KiB operand sections per step
  constexpr int NW = 4;                // waves (each loads and computes)
  constexpr int RBW = 4;               // 16-row blocks per wave
  constexpr int SPL = NSEC / NW;       // sections each wave loads per step
  static_assert(NSEC % NW == 0, "sections per wave");
  static_assert(NS >= 3 && NS <= 6, "ring stages");
  static_assert((NS - 1) * SPL < 64, "loads in flight per wave");
  static_assert(BS == 16 || BS == 32 || BS == 64, "block size");
  __shared__ u32x4 ring[NS][NSEC * 64];
  __shared__ int32_t blk_s[kMaxTreeBlocks];
  __shared__ TreeChunk ch_s[kMaxTreeChunks];

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
  for (int i = threadIdx.x; i < ti.n_blk; i += 256) blk_s[i] = sp.blk[ti.blk_off + i];
  {
    const int32_t* src = (const int32_t*)(sp.tchunks + ti.chunk_off);
    int32_t* dst = (int32_t*)ch_s;
    for (int i = threadIdx.x; i < ti.n_chunks * 12; i += 256) dst[i] = src[i];
  }
  __syncthreads();
  const bool rev = plane & 1;
  const int n_chunks = ti.n_chunks;
  const int total = ti.n_steps;

  auto enter = [&](Cursor& c, int i) __attribute__((always_inline)) {
    c.i = i;
    c.ci = rev ? n_chunks - 1 - i : i;
    c.s = 0;
    c.ntok = __builtin_amdgcn_readfirstlane(ch_s[c.ci].n_tok);
    c.nst = __builtin_amdgcn_readfirstlane(ch_s[c.ci].n_steps);
    c.blk = __builtin_amdgcn_readfirstlane(ch_s[c.ci].blk_off);
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
  // Sections wave + NW * k of the cursor's step into stage st: the first
  // SPL / 2 of a wave's sections are K (2KS = NSEC / 2 of them in all), the
  // rest V.
  auto issue = [&](const Cursor& c, int st) __attribute__((always_inline)) {
    const int tb = 32 * c.s;
    const int bA = blk_s[c.blk + tb / BS];
    const int bB = blk_s[c.blk + (tb + 16) / BS];
    const int64_t oA = (int64_t)bA * tile_step, oB = (int64_t)bB * tile_step;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int sect = wave + NW * k;
      const uint16_t* src;
      if (k < SPL / 2) {
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
    for (int k = SPL / 2; k < SPL; ++k) ring[st][(wave + NW * k) * 64 + lane] &= keep;
  };

  // ----------------------------------------------------------- queries
  // (rows past the item's last read the first holder's query; their
  // results are never written)
  bf16x8 qv[RBW][KS];
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    int row = 64 * wave + 16 * r + n;
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

  // ------------------------------------------------------------- math
  // One 32-token step of the chunk for this wave's four row blocks. Rows
  // outside the chunk's mask and tokens past its end get -inf scores
  // (full: no masking needed); blocks with no row in the mask skip their
  // products.
  auto math = [&](const u32x4* buf, uint64_t m64, int tb, int ntok, bool full, bool first_pass)
      __attribute__((always_inline)) {
    auto on = [&](int r) { return full || ((m64 >> (16 * r)) & 0xFFFFull) != 0; };
    uint32_t act[RBW];
#pragma unroll
    for (int r = 0; r < RBW; ++r) act[r] = __builtin_amdgcn_readfirstlane((int)(on(r) ? 1 : 0));
    u32x4 kreg[2 * KS], vreg[DB];
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) kreg[i] = buf[i * 64 + lane];
    f32x4 sc[RBW][2];
    float s8[RBW][8], mu[RBW];
    // scores of block r to masked, scaled maxima and the block's reference
    auto row_max = [&](int r) __attribute__((always_inline)) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) s8[r][4 * tau + i] = sc[r][tau][i];
      if (NEG) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s8[r][e] = -s8[r][e];
      }
      // (after the negation: a masked score stays -inf)
      if (!full) {
        const int valid = ((m64 >> (16 * r + n)) & 1ull) ? ntok - (tb + voff) : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) s8[r][e] = e < valid ? s8[r][e] : kNegInf;
      }
      float m = fmaxf(fmaxf(s8[r][0], s8[r][1]), fmaxf(s8[r][2], s8[r][3]));
      m = fmaxf(m, fmaxf(fmaxf(s8[r][4], s8[r][5]), fmaxf(s8[r][6], s8[r][7])));
      const float mx = max_xor32(max_xor16(m)) * cs;
      m_max[r] = fmaxf(m_max[r], mx);
      // the first finite maximum becomes the reference (nothing has been
      // accumulated yet, so nothing is rescaled)
      if (first_pass && m_ref[r] == kNegInf) m_ref[r] = mx;
      mu[r] = (m_ref[r] == kNegInf) ? 0.f : m_ref[r];
    };
    // block r + 1's products under block r's maxima
    qk_block<KS>(sc[0][0], sc[0][1], kreg, qv[0], act[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 1; r < RBW; ++r) {
      qk_block<KS>(sc[r][0], sc[r][1], kreg, qv[r], act[r]);
      __builtin_amdgcn_sched_barrier(0);
      row_max(r - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the V operands now (the K operands are dead): their reads overlap the
    // last block's maxima and the first probabilities
#pragma unroll
    for (int j = 0; j < DB; ++j) vreg[j] = buf[(2 * KS + j) * 64 + lane];
    settle_v(sc[RBW - 1][0], sc[RBW - 1][1]);
    row_max(RBW - 1);
    // block r's products, each followed by a slice of block r + 1's
    // probabilities (the next block's vector work under this block's
    // matrix products)
    Probs cur, nxt;
    cur.psum = 0.f;
    probs_slices<0, 8>(cur, s8[0], cs, mu[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
      nxt.psum = 0.f;
      const int rn = r + 1 < RBW ? r + 1 : r;
      if (r + 1 < RBW)
        pv_interleaved<0, DB, true>(acc[r], vreg, cur, nxt, s8[rn], cs, mu[rn], act[r]);
      else
        pv_interleaved<0, DB, false>(acc[r], vreg, cur, nxt, s8[rn], cs, mu[rn], act[r]);
      l_run[r] += cur.psum;
      cur = nxt;
    }
  };

  // -------------------------------------------------------------- loop
  // At step t: wait for this wave's loads of step t (the younger ones may
  // stay in flight), zero the ragged tail, barrier (step t has landed for
  // every wave, and every wave is done with step t - 1, whose stage is now
  // free), load step t + NS - 1 into that stage, compute step t. The
  // s_waitcnt immediate has vmcnt in bits 3:0 and 15:14; expcnt 7 and
  // lgkmcnt 15 mean no wait on those.
  constexpr int kWait = (NS - 2) * SPL;
  constexpr int kWaitVm = 0x0F70 | (kWait & 0xF) | ((kWait >> 4) << 14);
  __shared__ int redo_s;
#pragma unroll
  for (int r = 0; r < RBW; ++r) {
    m_ref[r] = kNegInf;
    m_max[r] = kNegInf;
  }
  for (int pass = 0; pass < 2; ++pass) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
#pragma unroll
      for (int j = 0; j < DB; ++j) zero_acc(acc[r][j], zero);
      l_run[r] = 0.f;
    }
    Cursor ld, cp;
    enter(ld, 0);
    enter(cp, 0);
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
      issue(ld, k);
      advance(ld);
    }
    int st_cur = 0, st_nxt = NS - 1;
    for (int t = 0; t < total; ++t) {
      __builtin_amdgcn_s_waitcnt(kWaitVm);
      if (cp.s == cp.nst - 1 && (cp.ntok & 31) != 0) zero_tail(cp, st_cur);
      __builtin_amdgcn_s_barrier();
      issue(ld, st_nxt);
      advance(ld);
      const uint64_t rows = ch_s[cp.ci].rows[wave];
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)rows);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(rows >> 32));
      const uint64_t m64 = ((uint64_t)hi << 32) | lo;
      const int tb = 32 * cp.s;
      if (m64 != 0) math(ring[st_cur], m64, tb, cp.ntok, m64 == ~0ull && tb + 32 <= cp.ntok, pass == 0);
      advance(cp);
      st_nxt = st_cur;
      st_cur = st_cur + 1 == NS ? 0 : st_cur + 1;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the walk

    // ---------------------------------------------------------- output
    bool bad = false;
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
      settle<DB>(acc[r]);
      const float l_tot = sum_xor32(sum_xor16(l_run[r]));
      const int row = 64 * wave + 16 * r + n;
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
  if (!tree_supported(D, BS) || (stages != 3 && stages != 4)) return hipErrorInvalidValue;
  if (n_wg <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_wg), block(256);
  const bool neg = p.q_flip != 0;  // a negative softmax scale
#define PKV_TREE_NS(d, bs, ns)                                                                   \
  return neg ? launch_kernel(attn_tree_kernel<d, bs, ns, true>, grid, block, stream, ev,         \
                             (const AttnCore&)p, p.meta)                                         \
             : launch_kernel(attn_tree_kernel<d, bs, ns, false>, grid, block, stream, ev,        \
                             (const AttnCore&)p, p.meta);
#define PKV_TREE(d, bs)               \
  if (D == d && BS == bs) {           \
    if (stages == 3) {                \
      PKV_TREE_NS(d, bs, 3)           \
    } else {                          \
      PKV_TREE_NS(d, bs, 4)           \
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
