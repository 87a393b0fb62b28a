// Launch wrappers for the device kernels in kernels.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_plan.h"

namespace pkv {

// Optional timing events: when set, the launch records them at the
// kernel's own start and end.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

constexpr int kInlineOps = 16;
constexpr int kInlineSlots = 64;

// One append: copy-on-write copies (ops: triples src, dst, n_valid) and the
// writes of n_slots new tokens ([L][n_slots][Hkv][D] K and V). Small lists
// travel inside the arguments (ops / slots == nullptr); larger ones are read
// from device memory.
struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* k_arena;
  void* v_arena;
  const int32_t* ops;
  const int64_t* slots;
  int32_t n_ops;
  int32_t n_slots;
  int32_t L;
  int32_t NB;
  int32_t Hkv;
  int32_t D;
  int32_t BS;
  int32_t pad;
  int32_t inl_ops[3 * kInlineOps];
  int64_t inl_slots[kInlineSlots];
};

hipError_t launch_append(int dtype, const AppendParams& p, hipStream_t stream,
                         const LaunchEvents& ev);

// True if the (dtype, D, BS) combination has a compiled attention kernel.
bool attn_supported(bool mfma, int dtype, int D, int BS);

// One workgroup per (work item, layer, KV head): grid = n_items * n_layers * Hkv.
// lo_split: P.V adds the bf16 rounding residual of P in a second product.
hipError_t launch_attn(bool mfma, bool lo_split, int dtype, int D, int BS, const AttnParams& p,
                       hipStream_t stream, const LaunchEvents& ev);

// max_entries: the longest per-branch list of partial states.
hipError_t launch_combine(int D, int max_entries, const CombineParams& p, hipStream_t stream,
                          const LaunchEvents& ev);

}  // namespace pkv
