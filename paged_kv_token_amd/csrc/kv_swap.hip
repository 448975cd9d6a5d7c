// Block swap between the device KV pools and a host tier ("Stateful Large Language Model
// Serving with Pensieve", Methodology: a GPU-CPU cache hierarchy whose tiers exchange cached
// KV tokens ahead of time, with the transfers pipelined behind computation).
//
// The host tier has the same block layout as the device pools; a swap copies whole blocks (all
// KV heads: one contiguous [Hkv][16][D] K run and one V run of the same layout per block).  Eight
// workgroups walk the (block, tensor) copies, each with 16-byte accesses that read or write the
// host tier directly through its device mapping: a batch of scattered blocks is one launch.  The
// copy is bound by the host link, and eight workgroups with eight 16-byte chunks in flight per
// thread (256 KB in all) keep it as busy as 128 workgroups did, while holding far fewer of the
// workgroup slots the attention kernels beside it need (13B step with a swap-in of 8.5 MB beside
// it: 0.386 ms with up to 128 workgroups, 0.345 ms with eight; 0.302 ms alone); four workgroups
// no longer fill the link.
#include "device_common.h"
#include "launch.h"

namespace pk {

// Copy `bytes` (a multiple of 16) with the workgroup's 256 threads, eight 16-byte chunks in flight
// per thread.
__device__ __forceinline__ void copy_run(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t bytes) {
  constexpr int U = 8;
  for (int64_t base = (int64_t)threadIdx.x * 16; base < bytes; base += 256 * 16 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = base + (int64_t)u * 256 * 16;
      if (off < bytes) v[u] = *reinterpret_cast<const u32x4*>(src + off);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = base + (int64_t)u * 256 * 16;
      if (off < bytes) *reinterpret_cast<u32x4*>(dst + off) = v[u];
    }
  }
}

__global__ __launch_bounds__(256) void kv_swap_kernel(const uint8_t* __restrict__ src_k,
                                                      const uint8_t* __restrict__ src_v, uint8_t* __restrict__ dst_k,
                                                      uint8_t* __restrict__ dst_v, const int32_t* __restrict__ pairs,
                                                      int n, int64_t block_bytes) {
  for (int job = blockIdx.x; job < 2 * n; job += gridDim.x) {
    const int i = job >> 1, tensor = job & 1;
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    const uint8_t* src = (tensor == 0 ? src_k : src_v) + s * block_bytes;
    uint8_t* dst = (tensor == 0 ? dst_k : dst_v) + d * block_bytes;
    copy_run(src, dst, block_bytes);
  }
}

hipError_t launch_kv_swap(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int32_t* pairs,
                          int n, int64_t block_bytes, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (block_bytes % 16 != 0) return hipErrorInvalidValue;
  const int grid = std::min(2 * n, 8);
  PK_LAUNCH(kv_swap_kernel, dim3(grid), dim3(256), stream, static_cast<const uint8_t*>(src_k),
            static_cast<const uint8_t*>(src_v), static_cast<uint8_t*>(dst_k), static_cast<uint8_t*>(dst_v), pairs, n,
            block_bytes);
  return hipGetLastError();
}

}  // namespace pk
