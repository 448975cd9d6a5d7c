// Upload of a host-built work list: a small kernel on the caller's stream copies it from the
// page-locked staging buffer (mapped into the device address space) into the workspace, so
// that the upload orders with the surrounding kernels inside one queue instead of handing
// over to a copy engine and back.  The host learns that a staging buffer may be refilled from
// per-workgroup flags the kernel stores into page-locked memory, not from an event: an event
// recorded between two kernels holds the next one back by a few microseconds.
#include "device_common.h"
#include "launch.h"

namespace pk {

__global__ __launch_bounds__(256) void stage_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int n, uint32_t* __restrict__ done, uint32_t seq) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) dst[i] = src[i];
  if (done) {
    // Every thread has stored what it loaded, so its reads of the host buffer are complete once
    // it reaches the barrier; one system-scope store then tells the host that this workgroup no
    // longer needs the buffer.
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(done + blockIdx.x, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

hipError_t launch_stage_copy(const void* src_mapped, void* dst, size_t bytes, hipStream_t stream, uint32_t* done,
                             uint32_t seq, int* blocks_out) {
  if (blocks_out) *blocks_out = 0;
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 != 0 || bytes / 16 > (size_t)INT32_MAX) return hipErrorInvalidValue;
  const int n = (int)(bytes / 16);
  const int blocks = std::min((n + 255) / 256, kStageCopyBlocks);
  hipLaunchKernelGGL(stage_copy_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src_mapped),
                     static_cast<u32x4*>(dst), n, done, seq);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess && blocks_out) *blocks_out = blocks;
  return e;
}

}  // namespace pk
