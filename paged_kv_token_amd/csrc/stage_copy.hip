// Upload of a host-built work list: a small kernel on the caller's stream copies it from the
// page-locked staging buffer (mapped into the device address space) into the workspace, so
// that the upload orders with the surrounding kernels inside one queue instead of handing
// over to a copy engine and back.
#include "device_common.h"
#include "launch.h"

namespace pk {

__global__ __launch_bounds__(256) void stage_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) dst[i] = src[i];
}

hipError_t launch_stage_copy(const void* src_mapped, void* dst, size_t bytes, hipStream_t stream, hipEvent_t done) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 != 0 || bytes / 16 > (size_t)INT32_MAX) return hipErrorInvalidValue;
  const int n = (int)(bytes / 16);
  const int blocks = std::min((n + 255) / 256, 64);
  if (done)   // the launch's own completion records `done`: no separate event packet in the queue
    hipExtLaunchKernelGGL(stage_copy_kernel, dim3(blocks), dim3(256), 0, stream, nullptr, done, 0,
                          static_cast<const u32x4*>(src_mapped), static_cast<u32x4*>(dst), n);
  else
    hipLaunchKernelGGL(stage_copy_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src_mapped),
                       static_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

}  // namespace pk
