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

// One append: copy-on-write copies and the writes of new tokens, whose K
// and V are [L][n_tok][Hkv][D]. An op is five ints: src, dst, n_valid,
// and the range [tok0, tok0 + m) of new tokens that land in dst right
// after the copied slots. The write list holds every other new token: its
// slot and its index in the new-token arrays. Small lists travel inside the
// arguments (ops / wslots / wtok == nullptr); larger ones are read from
// device memory.
struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* k_arena;
  void* v_arena;
  const int32_t* ops;
  const int64_t* wslots;
  const int32_t* wtok;
  int32_t n_ops;
  int32_t n_write;
  int32_t n_tok;
  int32_t L;
  int32_t NB;
  int32_t Hkv;
  int32_t D;
  int32_t BS;
  int32_t inl_ops[5 * kInlineOps];
  int64_t inl_slots[kInlineSlots];
  int32_t inl_tok[kInlineSlots];
};

// Reads the K/V of n tokens, given by slot (block * BS + offset), out of
// the arenas into rows row0 .. row0 + n - 1 of k_out / v_out, each
// [L][n_rows][Hkv][D] (the layout the append takes). At most kGatherSlots
// tokens per launch.
constexpr int kGatherSlots = 256;
struct GatherParams {
  const void* k_arena;
  const void* v_arena;
  void* k_out;
  void* v_out;
  int32_t n;        // tokens in this launch
  int32_t row0;     // their first row in the output
  int32_t n_rows;   // rows of the output ([L][n_rows][Hkv][D])
  int32_t L;
  int32_t NB;
  int32_t Hkv;
  int32_t D;
  int32_t BS;
  int64_t slots[kGatherSlots];
};

hipError_t launch_gather(int dtype, const GatherParams& p, hipStream_t stream,
                         const LaunchEvents& ev);

// Block sizes the append kernel is built for.
bool append_supported(int BS);

hipError_t launch_append(int dtype, const AppendParams& p, hipStream_t stream,
                         const LaunchEvents& ev);

// True if the (dtype, D, BS) combination has a compiled attention kernel.
bool attn_supported(bool mfma, int dtype, int D, int BS);

// One workgroup per entry of p.order (grid = p.n_order), each one (work
// item, layer, KV head). lo_split: P.V adds the bf16 rounding residual of P
// in a second product (the only form built).
// prefetch: each wave loads its next step while the current one computes
// (one row block per wave only). row_blocks_per_wave: 16-row blocks each
// wave of the matrix-core kernel owns, 1 or 2 (2 for D <= 128 only).
hipError_t launch_attn(bool mfma, bool lo_split, bool prefetch, int row_blocks_per_wave, int dtype,
                       int D, int BS, const AttnParams& p, hipStream_t stream,
                       const LaunchEvents& ev);

// The most 16-row blocks one wave of the matrix-core kernel can own at
// this head size.
int attn_max_row_blocks_per_wave(int D);

// The wide-row matrix-core kernel (bf16), same grid convention: waves per
// workgroup and 16-row blocks per wave, one of the compiled shapes
// (attn_wide_shape); a workgroup serves up to 16 * waves * row_blocks rows.
hipError_t launch_attn_wide(int D, int BS, int waves, int row_blocks, const AttnParams& p,
                            hipStream_t stream, const LaunchEvents& ev);

// The compiled wide shape for the requested one (in/out). waves counts the
// compute waves (4, 6 or 8; anything else: automatic, 8); row_blocks the
// 16-row blocks each owns (1 or 2; anything else: automatic, 2 up to
// head_dim 128 and 1 at 256). 6 waves, and 8 at head_dim 256, own one
// block each. The kernel adds its loader waves.
void attn_wide_shape(int D, int* waves, int* row_blocks);

// The wide kernel with specialised waves (wide_spec.hip): the same items,
// grid and partial states as launch_attn_wide, for head_dim 64 / 128 (bf16);
// each SIMD pairs a wave doing Q.K^T and the softmax with a wave doing P.V
// and the K/V loads. A workgroup serves up to spec_rows() rows (256).
bool spec_supported(int D, int BS);
int spec_rows();
hipError_t launch_attn_spec(int D, int BS, const AttnParams& p, hipStream_t stream,
                            const LaunchEvents& ev);

// The tree kernel (tree.hip): one workgroup per (tree item, layer, KV head)
// reads each chunk of the item once for all rows that hold it and writes
// the final output rows. stages: LDS ring depth (3 or 4). Built for bf16,
// head_dim 64 / 128 and block_size 16 / 32 / 64.
bool tree_supported(int D, int BS);
hipError_t launch_attn_tree(int D, int BS, int stages, const AttnParams& p, int n_wg,
                            hipStream_t stream, const LaunchEvents& ev);

// ------------------------------------------------------ static scratch
// Device memory for callers that cannot allocate (pkv_decode_attn_noalloc):
// a file-scope __device__ array of kScratchBytes in kernels.hip, one copy
// per GPU, held until the process ends. scratch_pointer returns its device
// address on the current device, looked up with hipGetSymbolAddress on the
// first call per device and kept (thread-safe).
constexpr size_t kScratchBytes = size_t(128) << 20;
hipError_t scratch_pointer(void** out);

// Writes n bytes from host memory to device memory dst through the launch
// arguments of a small copy kernel (kArgCopyBytes per launch, in stream
// order): no pinned staging buffer and no host-to-device copy command.
constexpr int kArgCopyBytes = 3072;
hipError_t launch_arg_copy(void* dst, const uint8_t* src, size_t n, hipStream_t stream);

// max_entries: the longest per-branch list of partial states.
hipError_t launch_combine(int D, int max_entries, const CombineParams& p, hipStream_t stream,
                          const LaunchEvents& ev);

}  // namespace pkv
