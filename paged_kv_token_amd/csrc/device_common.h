// Device helpers shared by the gfx950 kernels of libpensieve.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pk {

// kFP8: OCP E4M3 codes (pool storage only; decoded value times the pool's scale).
enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

template <int DT>
struct DTypeInfo {
  static constexpr int bytes = (DT == kF32) ? 4 : (DT == kFP8) ? 1 : 2;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One work item of an attention launch (32 bytes, planned on the host).
struct WorkItem {
  int32_t req;         // request index
  int32_t q_begin;     // first row of the item, relative to the request's first row
  int32_t q_count;     // rows (tokens) in the item
  int32_t kv_head;     // KV head g
  int32_t head_begin;  // first query head of the group handled (0..G-1)
  int32_t head_count;  // query heads of the group handled
  int32_t part;        // KV partition index
  int32_t num_parts;   // partitions of this request (1 = whole context, output goes to O)
};

// Arguments common to the attention kernels.
struct AttnArgs {
  const uint8_t* q;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;
  const int32_t* q_pos;      // may be null
  uint8_t* o;
  float* part_o;             // [rows][Hq][P][D] when items are split
  float* part_m;             // [rows][Hq][P]
  float* part_l;             // [rows][Hq][P]
  const int32_t* part_row_base;   // per request: partial row of its first query row (null: the query row itself)
  const WorkItem* items;
  int32_t num_items;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t bt_stride;
  int32_t part_stride;       // P of the partial buffers
  int32_t write_partials;    // 1: every item writes (m, l, O_p); 0: items with num_parts == 1 write O
  float scale;               // scale on q.k as stored (softmax scale times the K pool's scale)
  float scale_log2;          // scale * log2(e)
  float v_scale;             // scale of the V pool's stored values (1 for float pools)
};

// ---- element conversion ----------------------------------------------------
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Unpack one 16-byte chunk into 16 / bytes floats.
template <int DT>
__device__ __forceinline__ void unpack16(const u32x4 w, float* out) {
  if constexpr (DT == kF32) {
    // Copy each element to a scalar before the bit cast: hipcc (clang 22)
    // miscompiles __builtin_bit_cast applied directly to a vector-element
    // lvalue (it reads element 0 for every index).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t bits = w[i];
      out[i] = __builtin_bit_cast(float, bits);
    }
  } else if constexpr (DT == kF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = f16_bits_to_f32(w[i] & 0xFFFFu);
      out[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
    }
  } else if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      out[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
  } else {
    // E4M3 codes, decoded exactly by the hardware conversion (two per instruction).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = w[i];
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      out[4 * i] = lo[0];
      out[4 * i + 1] = lo[1];
      out[4 * i + 2] = hi[0];
      out[4 * i + 3] = hi[1];
    }
  }
}

// E4M3 code pair of two values already divided by the pool scale: magnitudes beyond 448 (the
// largest finite E4M3 value) saturate, NaN stays NaN, the rest round to nearest even.  The pair
// lands in the low (HI = false) or high half of `old`.
__device__ __forceinline__ float e4m3_saturate(float x) { return fabsf(x) > 448.f ? copysignf(448.f, x) : x; }
template <bool HI>
__device__ __forceinline__ uint32_t pack_e4m3x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_saturate(a), e4m3_saturate(b), (int)old, HI);
}

template <int DT>
__device__ __forceinline__ void store_elem(uint8_t* base, size_t index, float x) {
  if constexpr (DT == kF32) {
    reinterpret_cast<float*>(base)[index] = x;
  } else if constexpr (DT == kF16) {
    reinterpret_cast<uint16_t*>(base)[index] = f32_to_f16_bits(x);
  } else {
    reinterpret_cast<uint16_t*>(base)[index] = f32_to_bf16_bits(x);
  }
}

// ---- cross-lane reductions ---------------------------------------------------
// DPP controls (gfx9 encoding): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// Sum over aligned groups of N consecutive lanes (N = 1..64, power of two);
// every lane of a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f32<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp_f32<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f32<kDppRowMirror>(x);
  if constexpr (N >= 32) x += shfl_xor_f32(x, 16);
  if constexpr (N >= 64) x += shfl_xor_f32(x, 32);
  return x;
}

// Max over lanes that differ only in the bits selected by [FROM, 64): the
// lanes l, l ^ FROM, l ^ 2*FROM, ...  FROM is a power of two.
template <int FROM>
__device__ __forceinline__ float xor_max_from(float x) {
#pragma unroll
  for (int m = FROM; m < 64; m <<= 1) x = fmaxf(x, shfl_xor_f32(x, m));
  return x;
}

template <int FROM>
__device__ __forceinline__ float xor_sum_from(float x) {
#pragma unroll
  for (int m = FROM; m < 64; m <<= 1) x += shfl_xor_f32(x, m);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load of chunk `off` (bytes) of a tile through a buffer resource whose
// base is the wave-uniform tile address.  The offset VGPR is the only per-lane
// operand, so no 64-bit per-tile address is formed in VGPRs, and offsets at or
// beyond tile_bytes read as zero.  NT sets the load's non-temporal bit, for K/V
// that no other workgroup of the launch reads: the lines are not kept for reuse,
// and the loads-only stream of the 13B batch's K/V tiles runs 6.3 TB/s with it
// against 5.7 TB/s without (the same loads with the bit cost 10 % where several
// workgroups share a KV head's tiles through L2).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kAuxNonTemporal = 2;
template <bool NT = false>
__device__ __forceinline__ u32x4 tile_load16(const uint8_t* tile, uint32_t tile_bytes, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tile), (short)0, (int)tile_bytes, kBufferWord3);
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? kAuxNonTemporal : 0);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Block tables, lengths and work items are never written by a kernel that
// reads them; reading them through the constant address space lets uniform
// reads become scalar loads, which count on lgkmcnt instead of the in-order
// vector-memory counter that tracks the K/V stream.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ const_i32_ptr as_const(const int32_t* p) { return (const_i32_ptr)p; }

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum).  Placed once
// before a streaming loop: the compiler's wait-count tracking cannot prove at
// the loop header that loads issued before the loop (query rows, positions)
// have landed, and would otherwise wait on the vector-memory counter inside
// every iteration -- which, the counter being in order, also waits for the
// prefetch just issued for the next tile.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace pk
