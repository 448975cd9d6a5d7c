// Host-side launchers of the gfx950 kernels (one per kernel family).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace pk {

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                            const int32_t* slots, int num_tokens, int num_kv_heads, int head_dim,
                            int elem_bytes, hipStream_t stream);

// Vector-ALU attention: items of at most `rows_per_item` query vectors
// (tokens x heads of one KV group).  rows_per_item in {1, 2, 4, 8}.
hipError_t launch_attn_vector(const AttnArgs& args, int dtype, int head_dim, int rows_per_item,
                              hipStream_t stream);

// Matrix-core attention: items of up to 128 query vectors (tokens x the
// whole head group), fp16/bf16 only.
hipError_t launch_attn_mfma(const AttnArgs& args, int dtype, int head_dim, int group, hipStream_t stream);

// Merge of split partials into O: rows = partial rows x num_heads; rowmap
// (nullable) gives each partial row's output row and partition count.
hipError_t launch_split_merge(const float* part_o, const float* part_m, const float* part_l, int rows, int num_heads,
                              int head_dim, int num_partitions, const int32_t* rowmap, int dtype, void* o,
                              hipStream_t stream);

}  // namespace pk
