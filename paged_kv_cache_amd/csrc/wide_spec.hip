// Wide attention with specialised waves (gfx950, bf16 K/V, head_dim 64 or
// 128): the same work items, partial states and results as the wide kernel
// in kernels.hip (a chunk read by up to 256 query rows: the shared root of
// an MCTS tree), with the work of a step split between two kinds of wave.
//
// On this chip a SIMD does not overlap one wave's matrix products with that
// same wave's vector instructions, but it does overlap one wave's products
// with another wave's vector work. A wave that does both (the wide kernel's
// compute waves) runs products, then the softmax, then products again, and
// the step costs their sum. Here each SIMD holds a pair of waves serving the
// same four 16-row blocks (64 rows; four pairs, 256 rows):
//
//   softmax wave  Q.K^T of step i for its four blocks (each K operand read
//                 from LDS feeds four products), then the four blocks'
//                 softmax side by side: the reference moves (with its
//                 factor alpha per row) only when some lane's own maximum
//                 passes it by more than 8, the cross-lane row maximum is
//                 taken only then, and p = 2^(s c - m) goes to LDS as bf16
//                 hi + lo, with alpha;
//   P.V wave      in the same interval, P.V of step i - 1: per block the
//                 accumulators rescaled by alpha when some row moved its
//                 reference, then hi and lo products against each V
//                 operand read (each read feeds eight products), and two
//                 products against a ones operand that give the row sums.
//
// Each wave also moves a quarter of the operands the other wave of its pair
// reads from global memory into LDS (global_load_lds_dwordx4, in operand
// order, as the wide kernel's loader waves do): P.V waves the K sections,
// softmax waves the V sections, into two rings of five stages with three
// steps in flight. No wave reads the ring its own loads write, so the
// compiler (which makes a wave wait for its loads into LDS before it reads
// memory they may write) never holds a read behind loads still in flight.
// One barrier per step; P and alpha are double-buffered. Softmax waves take
// the lower wave ids, so that an arbiter favouring older waves starts a
// step's score products first.
//
// On the MCTS root this measures within 2% of the wide kernel (217.7 against
// 213.7-214.7 us), so it is an option (wide_spec), not the default: copies
// with parts removed put the loads and barriers alone at 106 us and the
// loads with the per-step LDS traffic (operand reads, the P exchange) at
// 168 us, with the softmax wave's chain on top.
//
// Numerics are the wide kernel's: scores unscaled until one FMA folds the
// scale into the exponent, the reference moved only when a row's maximum
// passes it by more than 8 (log2 units), P as bf16 plus its bf16 rounding
// residual (two products), fp32 accumulation; the partial state (m, l, acc)
// means out = acc / l with both scaled by 2^-m.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.h"
#include "kernels.hpp"

namespace pkv {

namespace {

constexpr int kPairs = 4;       // softmax waves = P.V waves = SIMDs
constexpr int kPairBlocks = 4;  // 16-row blocks per pair
constexpr int kStages = 5;      // K/V ring depth
constexpr int kAhead = 3;       // steps issued ahead of the one a wave reads

// A workgroup barrier the compiler may not move LDS accesses across (the
// ring is written by DMA, which it does not see). No hardware wait: each
// wave waits for its own traffic first where another wave reads it.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediates: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
constexpr int wait_vm(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }

template <int D, int BS>
__global__ __launch_bounds__(2 * kPairs * 64) void attn_spec_kernel(AttnCore p, PlanBytes plan_bytes) {
  constexpr int KS = D / 32;         // 32-deep slices of Q.K^T
  constexpr int DB = D / 16;         // 16-wide d blocks of P.V
  constexpr int NK = 2 * KS;         // K sections per step (two 16-token tiles)
  constexpr int NB = kPairs * kPairBlocks;
  constexpr int RB = kPairBlocks;
  constexpr int SPK = NK / kPairs;  // K sections each P.V wave loads per step
  constexpr int SPV = DB / kPairs;  // V sections each softmax wave loads per step
  static_assert(NK % kPairs == 0 && DB % kPairs == 0 && kAhead * SPV < 64, "loads in flight per wave");
  // a stage is refilled kAhead steps ahead: K(i + kAhead) over K(i + kAhead - kStages)
  // (read kStages - kAhead iterations ago), V likewise (read one iteration later)
  static_assert(kStages >= kAhead + 2, "ring depth");
  static_assert(BS == 16 || BS == 32 || BS == 64, "block size");
  __shared__ u32x4 ring_k[kStages][NK * 64];  // step i's K in stage i % kStages
  __shared__ u32x4 ring_v[kStages][DB * 64];  // step i's V in stage i % kStages
  __shared__ u32x4 pbuf[2][NB][2][64];  // per block: P hi, P lo (operand order)
  __shared__ float abuf[2][NB][64];     // per block: the rescale factor of each lane's row
  __shared__ int32_t blk_s[kMaxChunkBlocks];

  const PlanArrays sp = plan_arrays(p, plan_bytes);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool pv_wave = wave >= kPairs;
  const int pair = pv_wave ? wave - kPairs : wave;
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
  const int RBn = (it.n_rows + 15) >> 4;  // row blocks of the item
  // the pair's blocks are pair + kPairs * r; with any of them in the item
  // the pair computes all four (rows past the item have zero queries and
  // are never stored)
  const bool busy = pair < RBn;

  const uint16_t* K = (const uint16_t*)p.k_arena;
  const uint16_t* V = (const uint16_t*)p.v_arena;
  const int64_t layer_tiles = (int64_t)layer * p.num_blocks * p.Hkv;
  // Loads of step s: K sections pair + kPairs * i (P.V waves; section
  // (tau, ks): tile tau's 16 tokens, depth 32 ks .. 32 ks + 31) or V
  // sections (softmax waves; d block j). Lane l's 16 bytes land at l * 16
  // of the section, in the order the matrix product reads its operand.
  auto issue_k = [&](int s, u32x4* buf) __attribute__((always_inline)) {
    const int tbase = 32 * s;
    const int bA = blk_s[tbase / BS];
    const int bB = blk_s[(tbase + 16) / BS];
    const int koff0 = 8 * (n >> 2) + (n & 3);
#pragma unroll
    for (int i = 0; i < SPK; ++i) {
      const int sect = pair + kPairs * i;
      const int tau = sect / KS, ks = sect - (sect / KS) * KS;
      const int off = koff0 + 4 * tau;
      const int b = (BS == 16 && off >= 16) ? bB : bA;
      const uint16_t* src = K + ((layer_tiles + (int64_t)b * p.Hkv + kvh) * BS + (tbase + off) % BS) * D +
                            32 * ks + 8 * g;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)&buf[sect * 64], 16, 0, 0);
    }
  };
  auto issue_v = [&](int s, u32x4* buf) __attribute__((always_inline)) {
    const int tbase = 32 * s;
    const int b = blk_s[(tbase + voff) / BS];
#pragma unroll
    for (int i = 0; i < SPV; ++i) {
      const int j = pair + kPairs * i;
      const uint16_t* src = V + ((layer_tiles + (int64_t)b * p.Hkv + kvh) * D + 16 * j + n) * BS +
                            (tbase + voff) % BS;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)&buf[j * 64], 16, 0, 0);
    }
  };

  if (pv_wave) {
    f32x4 acc[RB][DB], lsum[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
#pragma unroll
      for (int j = 0; j < DB; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      lsum[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // a ones operand: every output row of its product is the row sum of P
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.f;

    // Iteration i: wait for this wave's K loads of step i (steps i + 1 ..
    // i + kAhead - 1 stay in flight), barrier, issue step i + kAhead's into
    // the stage that held step i + kAhead - kStages (read in an earlier
    // iteration), then P.V of step i - 1. Past the end the last step is
    // loaded again (in bounds, never read: into a stage other than the last
    // step's), so the count of younger loads stays the same.
#pragma unroll
    for (int a = 0; a < kAhead; ++a) issue_k(min(a, last), ring_k[a]);
    int st_issue = kAhead % kStages;
    for (int i = 0; i <= n_steps; ++i) {
      if (i <= last) __builtin_amdgcn_s_waitcnt(wait_vm((kAhead - 1) * SPK));
      step_barrier();
      issue_k(min(i + kAhead, last), ring_k[st_issue]);
      st_issue = st_issue == kStages - 1 ? 0 : st_issue + 1;
      if (i == 0 || !busy) continue;
      const int j = i - 1;
      const u32x4* st = ring_v[j % kStages];
      const int pb = j & 1;
      bf16x8 phi[RB], plo[RB];
      float al[RB];
      bool moved = false;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int b = pair + kPairs * r;
        al[r] = abuf[pb][b][lane];
        phi[r] = as_bf16x8(pbuf[pb][b][0][lane]);
        plo[r] = as_bf16x8(pbuf[pb][b][1][lane]);
        moved |= al[r] != 1.f;
      }
      if (__any(moved)) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
#pragma unroll
          for (int d = 0; d < DB; ++d) acc[r][d] *= al[r];
          lsum[r] *= al[r];
        }
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        lsum[r] = mfma_bf16(ones, phi[r], lsum[r]);
        lsum[r] = mfma_bf16(ones, plo[r], lsum[r]);
      }
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const bf16x8 a = as_bf16x8(st[d * 64 + lane]);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          acc[r][d] = mfma_bf16(a, phi[r], acc[r][d]);
          acc[r][d] = mfma_bf16(a, plo[r], acc[r][d]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (!busy) return;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = (pair + kPairs * r) * 16 + n;
      if (row >= it.n_rows) continue;
      const int64_t prow = (int64_t)(li * p.Hkv + kvh) * p.P + it.part_row + row;
      float* pa = p.part_acc + prow * D;
#pragma unroll
      for (int d = 0; d < DB; ++d) *(f32x4*)(pa + 16 * d + 4 * g) = acc[r][d];
      if (g == 0) p.part_ml[2 * prow + 1] = lsum[r][0];
    }
    return;
  }

  // ---- softmax wave
  const bool tree = it.mask_from != 0x7fffffff && it.t0 + it.n_tok > it.mask_from;
  bf16x8 qv[RB][KS];
  bool row_ok[RB];
  uint64_t anc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int row = (pair + kPairs * r) * 16 + n;
    row_ok[r] = row < it.n_rows;
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
  float m_run[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) m_run[r] = kNegInf;
  const float c = p.abs_scale_log2;
  // K sections in the order (ks, tau): consecutive reads alternate between
  // the two 16-token score tiles
  auto ksec = [](int i) { return (i & 1) * KS + (i >> 1); };

  // In the chunk's last step the V slots past its end may hold anything
  // (even NaN); each softmax wave zeroes them in the V sections it loaded,
  // after they land and before the barrier that hands them to the P.V
  // waves, so that 0 * V stays 0.
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
    for (int i = 0; i < SPV; ++i) cur[(pair + kPairs * i) * 64 + lane] &= keep;
  };

  // Iteration i: wait for this wave's V loads of step i - 1 (the P.V waves
  // read them in this iteration; steps i .. i + kAhead - 1 stay in flight),
  // barrier, issue step i + kAhead's V into the stage that held step
  // i + kAhead - kStages, then Q.K^T and the softmax of step i.
#pragma unroll
  for (int a = 0; a < kAhead; ++a) issue_v(min(a, last), ring_v[a]);
  int st_issue = kAhead % kStages;
  for (int i = 0; i <= n_steps; ++i) {
    if (i >= 1) {
      __builtin_amdgcn_s_waitcnt(wait_vm(kAhead * SPV));
      if (ragged && i - 1 == last) {
        zero_tail(ring_v[last % kStages]);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      }
    }
    step_barrier();
    issue_v(min(i + kAhead, last), ring_v[st_issue]);
    st_issue = st_issue == kStages - 1 ? 0 : st_issue + 1;
    if (i == n_steps || !busy) continue;
    const u32x4* st = ring_k[i % kStages];
    const int pb = i & 1;
    f32x4 sc4[RB][2];
#pragma unroll
    for (int r = 0; r < RB; ++r) sc4[r][0] = sc4[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const bf16x8 a = as_bf16x8(st[ksec(k) * 64 + lane]);
      const int tau = k & 1, ks = k >> 1;
#pragma unroll
      for (int r = 0; r < RB; ++r) sc4[r][tau] = mfma_bf16(a, qv[r][ks], sc4[r][tau]);
    }
    // The four blocks' softmax steps side by side (no branch between them),
    // so that one block's dependent chain of vector instructions fills the
    // latency of another's: one wave per SIMD does this work.
    const int tbase = 32 * i;
    const bool tail = tbase + 32 > it.n_tok;
    const int tv = tbase + voff;
    float sc[RB][8];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[r][4 * tau + e] = sc4[r][tau][e];
    if (tail || tree) {  // wave-uniform: only the chunk's last step and masked steps
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = tv + e;
          if (t >= it.n_tok) sc[r][e] = kNegInf;
          const int pos = it.t0 + t;
          if (tree && pos >= it.mask_from && !((anc[r] >> (pos - it.mask_from)) & 1ull))
            sc[r][e] = kNegInf;
        }
    }
    // The lazy reference moves only when a row's maximum passes it by more
    // than 8, so the row maxima across the four lanes of a row are taken
    // only when some lane's own maximum does (and on a row's first finite
    // scores, where the reference is -inf).
    float mx[RB], alpha[RB];
    bool any_need = false;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      mx[r] = rmax8_fresh(sc[r]) * c;
      any_need |= mx[r] > m_run[r] + 8.f;
      alpha[r] = 1.f;
    }
    if (__any(any_need)) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const float m_row = max_xor32(max_xor16(mx[r]));
        const bool need = m_row > m_run[r] + 8.f;
        const float m_new = need ? m_row : m_run[r];
        alpha[r] = need ? fast_exp2(m_run[r] - m_new) : 1.f;  // 0 on the first finite max
        m_run[r] = m_new;
      }
    }
    // p = 2^(s c - m) as bf16 hi + lo; the row sums come from the P.V
    // wave's products against a ones operand
    bf16x8 ph[RB], pl[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float m_use = (m_run[r] == kNegInf) ? 0.f : m_run[r];
      (void)probs8<true>(sc[r], c, m_use, ph[r], pl[r]);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int b = pair + kPairs * r;
      abuf[pb][b][lane] = alpha[r];
      pbuf[pb][b][0][lane] = __builtin_bit_cast(u32x4, ph[r]);
      pbuf[pb][b][1][lane] = __builtin_bit_cast(u32x4, pl[r]);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // P and alpha written before the next barrier
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (!busy) return;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if (!row_ok[r]) continue;
    const int row = (pair + kPairs * r) * 16 + n;
    const int64_t prow = (int64_t)(li * p.Hkv + kvh) * p.P + it.part_row + row;
    if (g == 0) p.part_ml[2 * prow] = m_run[r];
  }
}

}  // namespace

bool spec_supported(int D, int BS) {
  return (D == 64 || D == 128) && (BS == 16 || BS == 32 || BS == 64);
}

int spec_rows() { return 16 * kPairs * kPairBlocks; }

hipError_t launch_attn_spec(int D, int BS, const AttnParams& p, hipStream_t stream,
                            const LaunchEvents& ev) {
  if (!spec_supported(D, BS)) return hipErrorInvalidValue;
  if (p.n_order == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_order), block(2 * kPairs * 64);
#define PKV_SPEC(d, bs) \
  if (D == d && BS == bs) return launch_kernel(attn_spec_kernel<d, bs>, grid, block, stream, ev, (const AttnCore&)p, p.meta);
  PKV_SPEC(64, 16)
  PKV_SPEC(64, 32)
  PKV_SPEC(64, 64)
  PKV_SPEC(128, 16)
  PKV_SPEC(128, 32)
  PKV_SPEC(128, 64)
#undef PKV_SPEC
  return hipErrorInvalidValue;
}

}  // namespace pkv
