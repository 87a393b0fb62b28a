// A measuring aid beside the attention kernels: one pass of plain 16-byte
// vector loads over a device buffer, spread over every CU, timed by the
// caller to get the practical HBM read rate of the GPU (ordinary loads, and
// the non-temporal loads the attention kernels use for K/V that one wave
// reads). Not part of the cache or of attention.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.h"
#include "pkv.h"
#include "pool.hpp"

namespace pkv {

namespace {

// Reads n16 16-byte units once: each workgroup one contiguous range, its
// 256 lanes on consecutive units, four loads in flight per lane (a
// grid-strided form, every workgroup touching the whole buffer, read 6.1
// TB/s non-temporal against 7.1 for contiguous ranges). The loaded values
// feed a fold whose rare match writes the sink, so the loads stay.
template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* src, int64_t n16, uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  auto ld = [](const u32x4* p) { return NT ? __builtin_nontemporal_load(p) : *p; };
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = lo + threadIdx.x;
  for (; i + 768 < hi; i += 1024) {
    const u32x4 a = ld(src + i), b = ld(src + i + 256), c = ld(src + i + 512), d = ld(src + i + 768);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < hi; i += 256) acc ^= ld(src + i);
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) sink[blockIdx.x & 1023] = 1u;
}

}  // namespace

}  // namespace pkv

extern "C" int pkv_stream_read(const void* src, int64_t bytes, int32_t streaming, void* sink,
                               void* stream) {
  pkv::clear_error();
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 ||
      (streaming != 0 && streaming != 1))
    return pkv::fail(PKV_E_INVALID,
                     "stream_read: bytes must be a positive multiple of 16, src 16-byte aligned, "
                     "streaming 0 or 1");
  const dim3 grid(8192), block(256);
  const pkv::LaunchEvents none;
  const auto* s = (const pkv::u32x4*)src;
  hipError_t e = streaming
                     ? pkv::launch_kernel(pkv::stream_read_kernel<true>, grid, block, (hipStream_t)stream,
                                          none, s, bytes / 16, (uint32_t*)sink)
                     : pkv::launch_kernel(pkv::stream_read_kernel<false>, grid, block, (hipStream_t)stream,
                                          none, s, bytes / 16, (uint32_t*)sink);
  if (e != hipSuccess) return pkv::fail(PKV_E_HIP, std::string("stream read launch: ") + hipGetErrorString(e));
  return PKV_OK;
}
