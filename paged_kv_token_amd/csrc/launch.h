// Host-side launchers of the gfx950 kernels (one per kernel family).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace pk {

// Events the next kernel launch on this host thread records its start and end time into
// (through the dispatch packet itself, hipExtLaunchKernel); both null when not timing.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchEvents& launch_events();

// Launch a kernel on `stream`, timed into launch_events() when they are set (an ordinary
// launch otherwise).
#define PK_LAUNCH(KERNEL, GRID, BLOCK, STREAM, ...)                                                 \
  do {                                                                                             \
    const ::pk::LaunchEvents& pk_ev_ = ::pk::launch_events();                                      \
    if (pk_ev_.start)                                                                              \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, pk_ev_.start, pk_ev_.stop, 0, __VA_ARGS__); \
    else                                                                                           \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, __VA_ARGS__);                             \
  } while (0)

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                            const int32_t* slots, int num_tokens, int num_kv_heads, int head_dim,
                            int elem_bytes, hipStream_t stream);

// New f16 / bf16 K/V rows rounded to E4M3 codes (value / scale) into FP8 pools.
hipError_t launch_kv_append_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                const int32_t* slots, int num_tokens, int num_kv_heads, int head_dim, int src_dtype,
                                float k_scale, float v_scale, hipStream_t stream);

// Vector-ALU attention: items of at most `rows_per_item` query vectors
// (tokens x heads of one KV group).  rows_per_item in {1, 2, 4, 8}.
hipError_t launch_attn_vector(const AttnArgs& args, int dtype, int kv_dtype, int head_dim, int rows_per_item,
                              hipStream_t stream);

// Matrix-core attention: items of up to 128 query vectors (tokens x the
// whole head group) in four-wave workgroups, or with `wide` up to 256 in
// eight-wave workgroups (2-byte pools, or E4M3 pools at head_dim 128), fp16/bf16 queries.
hipError_t launch_attn_mfma(const AttnArgs& args, int dtype, int kv_dtype, int head_dim, int group, bool wide,
                            hipStream_t stream);

// Copy n whole blocks (K and V runs of block_bytes each) from src to dst pools; pairs holds n
// {source block, destination block} pairs.  Either side may be device-mapped host memory.
hipError_t launch_kv_swap(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int32_t* pairs,
                          int n, int64_t block_bytes, hipStream_t stream);

// Copy `bytes` (a multiple of 16) from a device-mapped page-locked host buffer to device
// memory with a kernel of at most kStageCopyBlocks workgroups on `stream`.  With `done` (a
// device-mapped page-locked array of kStageCopyBlocks words) each workgroup stores `seq` into
// done[its index] once its reads of the source are complete; *blocks_out (nullable) receives the
// number of workgroups launched.
constexpr int kStageCopyBlocks = 64;
hipError_t launch_stage_copy(const void* src_mapped, void* dst, size_t bytes, hipStream_t stream,
                             uint32_t* done = nullptr, uint32_t seq = 0, int* blocks_out = nullptr);

// Size of the library-owned device scratch of pensieve_attn_fwd_noalloc (one array per GPU).
constexpr size_t kScratchBytes = (size_t)64 << 20;

// Device address of this GPU's scratch array (looked up once per device, with that device
// current, and kept).
hipError_t scratch_for_current_device(void** ptr);

// Merge of split partials into O: rows = partial rows x num_heads; rowmap
// (nullable) gives each partial row's output row and partition count.
hipError_t launch_split_merge(const float* part_o, const float* part_m, const float* part_l, int rows, int num_heads,
                              int head_dim, int num_partitions, const int32_t* rowmap, int dtype, void* o,
                              hipStream_t stream);

}  // namespace pk
