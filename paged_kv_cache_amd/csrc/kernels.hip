// Device kernels of the paged KV cache, written for gfx950 (MI355X, wave64).
//
//   kv_write_kernel    scatter appended tokens' K/V into their slots
//   cow_copy_kernel    copy the valid slots of a shared tail block on write
//   attn_mfma_kernel   paged attention over shared tiles on the matrix cores
//                      (bf16 K/V and q, fp32 softmax and accumulation); with a
//                      draft-tree mask it is the verify kernel
//   attn_valu_kernel   the same work on the vector ALUs (fp32 or bf16 K/V)
//   combine_kernel     log-sum-exp merge of a row's partial states in
//                      logical order
//
// Layout: K tiles [BS][D] (token-major), V tiles [D][BS] (token index
// fastest). See include/pkv.h.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ u32x4 ld16(const void* ptr) { return *(const u32x4*)ptr; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) {
  return bf16_bits_to_f32(v);
}

// ------------------------------------------------------------- kv_write

template <typename T>
__global__ __launch_bounds__(256) void kv_write_kernel(const T* __restrict__ k_new,
                                                       const T* __restrict__ v_new, T* k_arena,
                                                       T* v_arena, const int64_t* __restrict__ slots,
                                                       int n, int L, int NB, int Hkv, int D,
                                                       int BS) {
  const int64_t total = (int64_t)L * n * Hkv * D;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = idx;
    const int d = (int)(r % D);
    r /= D;
    const int h = (int)(r % Hkv);
    r /= Hkv;
    const int i = (int)(r % n);
    const int l = (int)(r / n);
    const int64_t slot = slots[i];
    const int64_t blk = slot / BS;
    const int off = (int)(slot - blk * BS);
    const int64_t tile = ((int64_t)l * NB + blk) * Hkv + h;
    k_arena[(tile * BS + off) * D + d] = k_new[idx];
    v_arena[(tile * D + d) * BS + off] = v_new[idx];
  }
}

// ------------------------------------------------------------- cow_copy

// One workgroup per (op, layer, KV head): copies slots [0, n_valid) of the
// source tile into the destination tile, K and V.
template <typename T>
__global__ __launch_bounds__(256) void cow_copy_kernel(T* k_arena, T* v_arena,
                                                       const int32_t* __restrict__ ops, int L,
                                                       int NB, int Hkv, int D, int BS) {
  const int per_op = L * Hkv;
  const int o = blockIdx.x / per_op;
  const int rem = blockIdx.x - o * per_op;
  const int l = rem / Hkv, h = rem - (rem / Hkv) * Hkv;
  const int src = ops[3 * o], dst = ops[3 * o + 1], nv = ops[3 * o + 2];
  const int64_t st = ((int64_t)l * NB + src) * Hkv + h;
  const int64_t dt = ((int64_t)l * NB + dst) * Hkv + h;
  const int64_t tile = (int64_t)BS * D;
  // K: the first nv token rows are one contiguous run
  const T* ks = k_arena + st * tile;
  T* kd = k_arena + dt * tile;
  for (int i = threadIdx.x; i < nv * D; i += blockDim.x) kd[i] = ks[i];
  // V: nv leading entries of each of the D rows
  const T* vs = v_arena + st * tile;
  T* vd = v_arena + dt * tile;
  for (int i = threadIdx.x; i < nv * D; i += blockDim.x) {
    const int d = i / nv, t = i - (i / nv) * nv;
    vd[d * BS + t] = vs[d * BS + t];
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

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int BS>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnParams p) {
  constexpr int KS = D / 32;  // 32-wide k steps of Q.K
  constexpr int DB = D / 16;  // 16-wide d blocks of P.V
  constexpr int ACC_STRIDE = D + 4;
  static_assert(BS == 16 || BS == 32 || BS == 64, "block size");
  __shared__ float mrg_m[3][16];
  __shared__ float mrg_l[3][16];
  __shared__ float mrg_acc[3][16 * ACC_STRIDE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int per_item = p.n_layers * p.Hkv;
  const int item_idx = blockIdx.x / per_item;
  const int rem = blockIdx.x - item_idx * per_item;
  const int li = rem / p.Hkv;
  const int kvh = rem - li * p.Hkv;
  const int layer = p.layer0 + li;
  const WorkItem it = p.items[item_idx];

  const int RB = (it.n_rows + 15) >> 4;
  const int RBp = RB == 1 ? 1 : (RB == 2 ? 2 : 4);
  const int phases = 4 / RBp;
  const int rb = wave % RBp, phase = wave / RBp;
  const bool active = rb < RB;
  const int row = rb * 16 + n;
  const bool row_ok = active && row < it.n_rows;
  const int crow = it.r0 + row;
  const int hold = crow / p.G;
  const int gq = crow - hold * p.G;
  const int branch = row_ok ? p.holders[it.hold_off + hold] : 0;
  const int qh = kvh * p.G + gq;

  bf16x8 qv[KS];
  {
    const uint16_t* qp =
        (const uint16_t*)p.q + (((int64_t)li * p.n_branch + branch) * p.Hq + qh) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok) raw = ld16(qp + 32 * ks);
      qv[ks] = as_bf16x8(raw);
    }
  }
  const bool tree = it.mask_from != 0x7fffffff && it.t0 + it.n_tok > it.mask_from;
  const uint64_t anc = (tree && row_ok) ? p.anc[branch] : ~0ull;

  const uint16_t* K = (const uint16_t*)p.k_arena;
  const uint16_t* V = (const uint16_t*)p.v_arena;
  const int64_t layer_tiles = (int64_t)layer * p.num_blocks * p.Hkv;
  const int32_t* blk = p.blk + it.blk_off;

  f32x4 acc[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  const int n_steps = (it.n_tok + 31) >> 5;

  if (active) {
    for (int s = phase; s < n_steps; s += phases) {
      const int tbase = s * 32;
      // scores: two S^T tiles of 16 tokens
      f32x4 st[2];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int tk = tbase + 8 * (n >> 2) + 4 * tau + (n & 3);
        const int b = blk[tk / BS];
        const uint16_t* kp = K + ((layer_tiles + (int64_t)b * p.Hkv + kvh) * BS + (tk % BS)) * D + 8 * g;
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) c = mfma_bf16(as_bf16x8(ld16(kp + 32 * ks)), qv[ks], c);
        st[tau] = c;
      }
      // V^T operands: 8 tokens (8g .. 8g+7 of the step) of d = 16 j + n
      const int tv = tbase + 8 * g;
      const int bv = blk[tv / BS];
      const uint16_t* vp = V + ((layer_tiles + (int64_t)bv * p.Hkv + kvh) * D + n) * BS + (tv % BS);
      u32x4 vraw[DB];
#pragma unroll
      for (int j = 0; j < DB; ++j) vraw[j] = ld16(vp + (int64_t)16 * j * BS);

      const bool tail = tbase + 32 > it.n_tok;
      float sc[8];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * tau + i;
          const int t = tv + e;
          float v = st[tau][i] * p.scale_log2;
          if (tail && t >= it.n_tok) v = kNegInf;
          if (tree) {
            const int pos = it.t0 + t;
            if (pos >= it.mask_from && !((anc >> (pos - it.mask_from)) & 1ull)) v = kNegInf;
          }
          sc[e] = v;
        }
      if (tail) {
        // slots past the chunk may hold anything (even NaN): zero them so
        // that 0 * V stays 0 in the P.V product
        u32x4 keep;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = (tv + 2 * w < it.n_tok) ? 0x0000ffffu : 0u;
          const uint32_t hi = (tv + 2 * w + 1 < it.n_tok) ? 0xffff0000u : 0u;
          keep[w] = lo | hi;
        }
#pragma unroll
        for (int j = 0; j < DB; ++j) vraw[j] &= keep;
      }

      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float psum = 0.f;
      bf16x8 phi, plo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = fast_exp2(sc[e] - m_use);
        psum += pe;
        const __bf16 h = (__bf16)pe;
        phi[e] = h;
        plo[e] = (__bf16)(pe - (float)h);
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < DB; ++j) {
        acc[j] *= alpha;
        acc[j] = mfma_bf16(as_bf16x8(vraw[j]), phi, acc[j]);
        acc[j] = mfma_bf16(as_bf16x8(vraw[j]), plo, acc[j]);
      }
    }
  }
  // the four lane groups hold disjoint tokens of the same rows
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);

  if (phases > 1) {
    if (phase > 0 && active) {
      const int slot = (phase - 1) * RBp + rb;
      if (g == 0) {
        mrg_m[slot][n] = m_run;
        mrg_l[slot][n] = l_tot;
      }
#pragma unroll
      for (int j = 0; j < DB; ++j)
        *(f32x4*)&mrg_acc[slot][n * ACC_STRIDE + 16 * j + 4 * g] = acc[j];
    }
    __syncthreads();
    if (phase == 0 && active) {
      for (int ph = 1; ph < phases; ++ph) {
        const int slot = (ph - 1) * RBp + rb;
        const float mo = mrg_m[slot][n], lo = mrg_l[slot][n];
        const float M = fmaxf(m_run, mo);
        if (M != kNegInf) {
          const float a = fast_exp2(m_run - M), b = fast_exp2(mo - M);
          l_tot = l_tot * a + lo * b;
#pragma unroll
          for (int j = 0; j < DB; ++j) {
            const f32x4 o = *(const f32x4*)&mrg_acc[slot][n * ACC_STRIDE + 16 * j + 4 * g];
            acc[j] = acc[j] * a + o * b;
          }
          m_run = M;
        }
      }
    }
  }
  if (phase == 0 && row_ok) {
    const int64_t prow = (int64_t)(li * p.Hkv + kvh) * p.P + it.part_row + row;
    if (g == 0) {
      p.part_ml[2 * prow] = m_run;
      p.part_ml[2 * prow + 1] = l_tot;
    }
    float* pa = p.part_acc + prow * D;
#pragma unroll
    for (int j = 0; j < DB; ++j) *(f32x4*)(pa + 16 * j + 4 * g) = acc[j];
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
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnParams p) {
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
  const int per_item = p.n_layers * p.Hkv;
  const int item_idx = blockIdx.x / per_item;
  const int rem = blockIdx.x - item_idx * per_item;
  const int li = rem / p.Hkv;
  const int kvh = rem - li * p.Hkv;
  const int layer = p.layer0 + li;
  const WorkItem it = p.items[item_idx];
  const int nr = it.n_rows;

  const T* Q = (const T*)p.q;
  for (int idx = threadIdx.x; idx < nr * D; idx += blockDim.x) {
    const int r = idx / D, d = idx - (idx / D) * D;
    const int crow = it.r0 + r;
    const int hold = crow / p.G, gq = crow - (crow / p.G) * p.G;
    const int branch = p.holders[it.hold_off + hold];
    qs[r][d] = to_f32<T>(Q[(((int64_t)li * p.n_branch + branch) * p.Hq + kvh * p.G + gq) * D + d]);
  }
  __syncthreads();

  const T* K = (const T*)p.k_arena;
  const T* V = (const T*)p.v_arena;
  const int64_t layer_tiles = (int64_t)layer * p.num_blocks * p.Hkv;
  const int32_t* blk = p.blk + it.blk_off;
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
// One workgroup per (layer, branch, KV head): for each of the G query heads
// and each d, merge the branch's partial states in logical order:
//   M = max m_i, L = sum l_i 2^(m_i - M), out = sum acc_i 2^(m_i - M) / L.

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int per = p.n_branch * p.Hkv;
  const int li = blockIdx.x / per;
  const int rem = blockIdx.x - li * per;
  const int b = rem / p.Hkv;
  const int kvh = rem - b * p.Hkv;
  const int e0 = p.comb_ptr[b], e1 = p.comb_ptr[b + 1];
  const int64_t plane = (int64_t)(li * p.Hkv + kvh) * p.P;
  for (int idx = threadIdx.x; idx < p.G * D; idx += blockDim.x) {
    const int gq = idx / D, d = idx - (idx / D) * D;
    float M = kNegInf;
    for (int e = e0; e < e1; ++e) M = fmaxf(M, p.part_ml[2 * (plane + p.comb_rows[e] + gq)]);
    float L = 0.f, O = 0.f;
    for (int e = e0; e < e1; ++e) {
      const int64_t row = plane + p.comb_rows[e] + gq;
      const float mi = p.part_ml[2 * row];
      if (mi == kNegInf) continue;
      const float w = fast_exp2(mi - M);
      L += p.part_ml[2 * row + 1] * w;
      O += p.part_acc[row * D + d] * w;
    }
    p.out[(((int64_t)li * p.n_branch + b) * p.Hq + kvh * p.G + gq) * D + d] = O / L;
  }
}

// ------------------------------------------------------------- launchers

hipError_t launch_kv_write(int dtype, const void* k_new, const void* v_new, void* k_arena,
                           void* v_arena, const int64_t* d_slots, int n, int L, int NB, int Hkv,
                           int D, int BS, hipStream_t stream) {
  const int64_t total = (int64_t)L * n * Hkv * D;
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 65536 ? want : 65536);
  if (dtype == 0)
    kv_write_kernel<float><<<grid, 256, 0, stream>>>((const float*)k_new, (const float*)v_new,
                                                     (float*)k_arena, (float*)v_arena, d_slots, n,
                                                     L, NB, Hkv, D, BS);
  else
    kv_write_kernel<uint16_t><<<grid, 256, 0, stream>>>(
        (const uint16_t*)k_new, (const uint16_t*)v_new, (uint16_t*)k_arena, (uint16_t*)v_arena,
        d_slots, n, L, NB, Hkv, D, BS);
  return hipGetLastError();
}

hipError_t launch_cow_copy(int dtype, void* k_arena, void* v_arena, const int32_t* d_ops,
                           int n_ops, int L, int NB, int Hkv, int D, int BS, hipStream_t stream) {
  if (n_ops == 0) return hipSuccess;
  const int grid = n_ops * L * Hkv;
  if (dtype == 0)
    cow_copy_kernel<float><<<grid, 256, 0, stream>>>((float*)k_arena, (float*)v_arena, d_ops, L,
                                                     NB, Hkv, D, BS);
  else
    cow_copy_kernel<uint16_t><<<grid, 256, 0, stream>>>((uint16_t*)k_arena, (uint16_t*)v_arena,
                                                        d_ops, L, NB, Hkv, D, BS);
  return hipGetLastError();
}

bool attn_supported(bool mfma, int dtype, int D, int BS) {
  const bool shape_ok = (D == 64 || D == 128 || D == 256) && (BS == 16 || BS == 32 || BS == 64);
  if (!shape_ok) return false;
  if (mfma) return dtype == 1;
  return dtype == 0 || dtype == 1;
}

#define PKV_DISPATCH_BS(KERNEL_T, ...)                                        \
  switch (BS) {                                                               \
    case 16: KERNEL_T(16)<<<grid, 256, 0, stream>>>(__VA_ARGS__); break;      \
    case 32: KERNEL_T(32)<<<grid, 256, 0, stream>>>(__VA_ARGS__); break;      \
    default: KERNEL_T(64)<<<grid, 256, 0, stream>>>(__VA_ARGS__); break;      \
  }

hipError_t launch_attn(bool mfma, int dtype, int D, int BS, const AttnParams& p,
                       hipStream_t stream) {
  if (!attn_supported(mfma, dtype, D, BS)) return hipErrorInvalidValue;
  const int64_t g64 = (int64_t)p.n_items * p.n_layers * p.Hkv;
  if (g64 == 0) return hipSuccess;
  if (g64 > 0x7fffffff) return hipErrorInvalidValue;
  const int grid = (int)g64;
  if (mfma) {
#define K_MFMA_64(bs) attn_mfma_kernel<64, bs>
#define K_MFMA_128(bs) attn_mfma_kernel<128, bs>
#define K_MFMA_256(bs) attn_mfma_kernel<256, bs>
    if (D == 64) {
      PKV_DISPATCH_BS(K_MFMA_64, p)
    } else if (D == 128) {
      PKV_DISPATCH_BS(K_MFMA_128, p)
    } else {
      PKV_DISPATCH_BS(K_MFMA_256, p)
    }
  } else if (dtype == 0) {
#define K_VF_64(bs) attn_valu_kernel<float, 64, bs>
#define K_VF_128(bs) attn_valu_kernel<float, 128, bs>
#define K_VF_256(bs) attn_valu_kernel<float, 256, bs>
    if (D == 64) {
      PKV_DISPATCH_BS(K_VF_64, p)
    } else if (D == 128) {
      PKV_DISPATCH_BS(K_VF_128, p)
    } else {
      PKV_DISPATCH_BS(K_VF_256, p)
    }
  } else {
#define K_VB_64(bs) attn_valu_kernel<uint16_t, 64, bs>
#define K_VB_128(bs) attn_valu_kernel<uint16_t, 128, bs>
#define K_VB_256(bs) attn_valu_kernel<uint16_t, 256, bs>
    if (D == 64) {
      PKV_DISPATCH_BS(K_VB_64, p)
    } else if (D == 128) {
      PKV_DISPATCH_BS(K_VB_128, p)
    } else {
      PKV_DISPATCH_BS(K_VB_256, p)
    }
  }
  return hipGetLastError();
}

hipError_t launch_combine(int D, const CombineParams& p, hipStream_t stream) {
  const int64_t g64 = (int64_t)p.n_layers * p.n_branch * p.Hkv;
  if (g64 == 0) return hipSuccess;
  const int grid = (int)g64;
  if (D == 64)
    combine_kernel<64><<<grid, 256, 0, stream>>>(p);
  else if (D == 128)
    combine_kernel<128><<<grid, 256, 0, stream>>>(p);
  else if (D == 256)
    combine_kernel<256><<<grid, 256, 0, stream>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
