// Launch wrappers for the device kernels in kernels.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_plan.h"

namespace pkv {

// Scatter n tokens of new K/V ([L][n][Hkv][D]) into their slots.
hipError_t launch_kv_write(int dtype, const void* k_new, const void* v_new, void* k_arena,
                           void* v_arena, const int64_t* d_slots, int n, int L, int NB, int Hkv,
                           int D, int BS, hipStream_t stream);

// Copy-on-write: d_ops holds n_ops triples (src, dst, n_valid).
hipError_t launch_cow_copy(int dtype, void* k_arena, void* v_arena, const int32_t* d_ops,
                           int n_ops, int L, int NB, int Hkv, int D, int BS, hipStream_t stream);

// True if the (dtype, D, BS) combination has a compiled attention kernel.
bool attn_supported(bool mfma, int dtype, int D, int BS);

// One workgroup per (work item, layer, KV head): grid = n_items * n_layers * Hkv.
hipError_t launch_attn(bool mfma, int dtype, int D, int BS, const AttnParams& p,
                       hipStream_t stream);

// One workgroup per (layer, branch, KV head).
hipError_t launch_combine(int D, const CombineParams& p, hipStream_t stream);

}  // namespace pkv
