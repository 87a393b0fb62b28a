// Device helpers shared by the attention kernels (kernels.hip, tree.hip):
// vector types, loads, the gfx950 row-swap reductions, the bf16 matrix-core
// product, the plan arrays and the online-softmax pieces. gfx950 (wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_plan.h"
#include "kernels.hpp"

namespace pkv {

// Launches a kernel; with timing events, through the HIP extension that
// records them when the kernel itself starts and ends.
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                                const LaunchEvents& ev, Args... args) {
  if (ev.start)
    hipExtLaunchKernelGGL(kern, grid, block, 0, stream, ev.start, ev.stop, 0, args...);
  else
    kern<<<grid, block, 0, stream>>>(args...);
  return hipGetLastError();
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ u32x4 ld16(const void* ptr) { return *(const u32x4*)ptr; }

// K/V tiles that only one wave reads are fetched with streaming
// (non-temporal) loads: on gfx950 they sustain ~7 TB/s on long reads where
// ordinary loads stop near 5.4 TB/s. Tiles that two waves of a workgroup,
// or sibling workgroups, read use ordinary loads, so that the second read
// hits in the caches instead of going back to HBM.
__device__ __forceinline__ u32x4 ld16_stream(const void* ptr) {
  return __builtin_nontemporal_load((const u32x4*)ptr);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 row-swap permutes. v_permlane16_swap exchanges the
// odd rows of its first register with the even rows of its second, and
// v_permlane32_swap the upper half of the first with the lower half of the
// second; starting from two copies of x, each lane then holds its own and
// its partner's value in the two registers. Written as one asm statement
// with both registers as in/out operands, preceded by the two wait states
// the permute needs after the VALU write of its operands.
__device__ __forceinline__ void swap16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// Maxima as written (v_max_f32, v_max3_f32): on values the compiler cannot
// prove canonical (results of asm statements and matrix products, lanes
// moved by the permutes) fmaxf quiets each input first, two more vector
// instructions per maximum. Quiet NaN inputs are ignored as by fmaxf.
__device__ __forceinline__ float rmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float rmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float rmax8(const float (&x)[8]) {
  return rmax(rmax3(x[0], x[1], x[2]), rmax3(x[3], x[4], rmax3(x[5], x[6], x[7])));
}
// rmax8 of values that may come straight from matrix products: the compiler
// does not add the wait states a product's result needs before a vector
// instruction reads it when the reader is an asm statement, so the statement
// waits them itself (s_nop 7: the 8 the compiler gives its own readers of a
// v_mfma_f32_16x16x32_bf16 result).
__device__ __forceinline__ float rmax8_fresh(const float (&x)[8]) {
  float a, b;
  asm("s_nop 7\n\t"
      "v_max3_f32 %0, %2, %3, %4\n\t"
      "v_max3_f32 %1, %5, %6, %7\n\t"
      "v_max3_f32 %0, %0, %8, %9\n\t"
      "v_max_f32 %0, %0, %1"
      : "=&v"(a), "=&v"(b)
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
  return a;
}
__device__ __forceinline__ float max_xor16(float x) {
  float a = x, b = x;
  swap16(a, b);
  return rmax(a, b);
}
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  swap32(a, b);
  return rmax(a, b);
}
__device__ __forceinline__ float sum_xor16(float x) {
  float a = x, b = x;
  swap16(a, b);
  return a + b;
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a = x, b = x;
  swap32(a, b);
  return a + b;
}

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

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The schedule's arrays, from the launch's own arguments or from the
// workspace. Both bases are global memory (kernel arguments live there
// too), which the casts tell the compiler so that every read of the
// schedule stays a global (or scalar) load.
struct PlanArrays {
  const WorkItem* items;
  const int32_t* blk;
  const int32_t* holders;
  const uint64_t* anc;
  const int32_t* order;
  const int32_t* comb_ptr;
  const int32_t* comb_rows;
  const TreeItem* titems;
  const TreeChunk* tchunks;
  const int32_t* binfo;
};
typedef const __attribute__((address_space(1))) uint8_t* gbytes_t;
__device__ __forceinline__ PlanArrays plan_arrays(const AttnCore& p, const PlanBytes& m) {
  const gbytes_t b = p.meta_inline ? (gbytes_t)(const uint8_t*)m.b : (gbytes_t)p.meta_dev;
  return {(const WorkItem*)(b + p.off_items),     (const int32_t*)(b + p.off_blk),
          (const int32_t*)(b + p.off_holders),    (const uint64_t*)(b + p.off_anc),
          (const int32_t*)(b + p.off_order),      (const int32_t*)(b + p.off_comb_ptr),
          (const int32_t*)(b + p.off_comb_rows),  (const TreeItem*)(b + p.off_titems),
          (const TreeChunk*)(b + p.off_tchunks),  (const int32_t*)(b + p.off_binfo)};
}

// Online softmax with a lazy reference: a row's probabilities are taken as
// 2^(s - m) against a reference m that is moved (and the running sum and
// accumulators rescaled) only when the row's maximum exceeds it by more
// than 8, so weights stay below 2^8 and the accumulators, which live in
// AGPRs, are rarely touched outside the matrix products. The vote keeps the
// branch wave-uniform. The partial state (m, l, acc) then means
// out = acc / l with acc and l both scaled by 2^-m, as before.
template <int DB>
__device__ __forceinline__ void rebase(float mx, float& m_ref, float& l_run, f32x4 (&acc)[DB]) {
  const bool need = mx > m_ref + 8.f;
  if (__any(need)) {
    const float m_new = need ? mx : m_ref;
    const float alpha = need ? fast_exp2(m_ref - m_new) : 1.f;  // 0 on the first finite max
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < DB; ++j) acc[j] *= alpha;
    m_ref = m_new;
  }
}

// Probabilities of one 16-row block's eight scores per lane: p = 2^(s c - m)
// with the scale c folded into one FMA (scores stay unscaled until here),
// converted to bf16 two at a time (v_cvt_pk_bf16_f32), with LO the bf16
// rounding residual p - bf16(p) as well. Returns the lane's sum of p. Used
// by the wide kernel, whose math bounds it (MCTS root 228 -> 221 us, verify
// 280 -> 277 us); in the memory-bound narrow kernel the same change measured
// 1-1.5% slower, so it keeps the scaled-score form.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <bool LO>
__device__ __forceinline__ float probs8(const float (&sc)[8], float c, float m_use, bf16x8& phi,
                                        bf16x8& plo) {
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float p0 = fast_exp2(__builtin_fmaf(sc[e], c, -m_use));
    const float p1 = fast_exp2(__builtin_fmaf(sc[e + 1], c, -m_use));
    psum += p0 + p1;
    const bf16x2 h = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
    phi[e] = h[0];
    phi[e + 1] = h[1];
    if (LO) {
      const f32x2 hf = __builtin_convertvector(h, f32x2);
      const bf16x2 l = __builtin_convertvector((f32x2){p0 - hf[0], p1 - hf[1]}, bf16x2);
      plo[e] = l[0];
      plo[e + 1] = l[1];
    }
  }
  return psum;
}

// A chunk's block ids are copied to LDS when the workgroup starts (at most
// kMaxChunkBlocks of them; the planner cuts chunks to fit) and read from
// there at wave-uniform indexes. Read from global memory as each step
// needs them, they would be vector loads (the compiler cannot prove the
// table unwritten, so it does not use the scalar cache) with a wait in
// front of every step, and that wait would also drain the K/V loads
// already in flight.
template <int BS>
__device__ __forceinline__ int stage_block_ids(int32_t* dst, const int32_t* blk, int n_steps) {
  const int nbk = (32 * n_steps + BS - 1) / BS;
  for (int i = threadIdx.x; i < nbk; i += blockDim.x) dst[i] = blk[i];
  return nbk;
}

}  // namespace pkv
