// KV append: slot-mapped copy of new K/V rows into the paged pools.
//
// A token's slot is physical_block * 16 + offset: the block the caller
// allocated for it ("LLM上下文缓存与状态复用机制的分析和探索", section 3.1:
// fixed-size blocks allocated on demand in non-contiguous memory).
//
// Both pools are [num_blocks][Hkv][16][D]: a token's row for one KV head is D
// contiguous elements, so every row leaves in whole 16-byte stores and covers
// whole cache lines (256 bytes at f16 / bf16, D = 128); no partly written
// sector is left for a read-modify-write when it leaves the caches.  The first
// half of the grid copies K, the second V: thread i of a half copies 16-byte
// chunk i % CPR of row i / CPR (token, KV head), so consecutive threads read
// consecutive bytes of the [N][Hkv][D] inputs and write consecutive bytes of
// each destination row (one 16-byte load and store per thread measured 2-5 %
// faster than one thread copying the same chunk of both tensors).
//
// Loads and stores are non-temporal: the new rows are read once and the pool rows are not read
// again in this kernel, so they go past the caches instead of leaving dirty lines there for the
// next kernel (the attention over the same pools) to write back while it streams.  Measured on
// the 13B batch: the matrix-core launch after the append 0.203 -> 0.188 ms, the step
// 0.364 -> 0.350 ms.
#include "device_common.h"
#include "launch.h"

namespace pk {

template <int EB, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
                                                        uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                        const int32_t* __restrict__ slots, int num_tokens,
                                                        int num_kv_heads) {
  constexpr int ROW = D * EB;        // bytes of one token's row for one head
  constexpr int CPR = ROW / 16;      // 16-byte chunks per row
  const uint32_t total = (uint32_t)num_tokens * (uint32_t)num_kv_heads * CPR;   // chunks per tensor
  uint32_t i = blockIdx.x * 256u + threadIdx.x;   // the launch keeps 2 * total + 255 below 2^31
  if (i >= 2 * total) return;
  const bool isv = i >= total;
  if (isv) i -= total;
  const uint32_t c = i % CPR;
  const uint32_t row = i / CPR;               // token * Hkv + head
  const uint32_t t = row / (uint32_t)num_kv_heads, g = row % (uint32_t)num_kv_heads;
  // The new row is read before the slot is tested: chunk i is in bounds whatever the slot holds,
  // and both loads are then in flight together instead of one after the other.  The empty asm
  // statement (no instruction) takes the row as an operand before the test, so the compiler
  // cannot sink its load below it.
  u32x4 x = __builtin_nontemporal_load((isv ? v_new : k_new) + i);
  const int s = slots[t];
  asm volatile("" : "+v"(x));
  if (s < 0) return;
  const size_t dst = (((size_t)(s >> 4) * num_kv_heads + g) * 16 + (size_t)(s & 15)) * ROW + (size_t)c * 16;
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>((isv ? v_pool : k_pool) + dst));
}

template <int EB, int D>
static hipError_t launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                const int32_t* slots, int num_tokens, int num_kv_heads, hipStream_t stream) {
  constexpr int CPR = D * EB / 16;
  const long long chunks = (long long)num_tokens * num_kv_heads * CPR;
  if (2 * chunks + 255 > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)((2 * chunks + 255) / 256));
  PK_LAUNCH((kv_append_kernel<EB, D>), grid, dim3(256), stream, static_cast<const u32x4*>(k_new),
            static_cast<const u32x4*>(v_new), static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), slots,
            num_tokens, num_kv_heads);
  return hipGetLastError();
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                            const int32_t* slots, int num_tokens, int num_kv_heads, int head_dim,
                            int elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  if (elem_bytes == 4) {
    return head_dim == 64 ? launch_append<4, 64>(k_new, v_new, k_pool, v_pool, slots, num_tokens, num_kv_heads, stream)
                          : launch_append<4, 128>(k_new, v_new, k_pool, v_pool, slots, num_tokens, num_kv_heads, stream);
  }
  return head_dim == 64 ? launch_append<2, 64>(k_new, v_new, k_pool, v_pool, slots, num_tokens, num_kv_heads, stream)
                        : launch_append<2, 128>(k_new, v_new, k_pool, v_pool, slots, num_tokens, num_kv_heads, stream);
}

// FP8 append ("LLM上下文缓存与状态复用机制的分析和探索", section 4(3): the KV cache stored as
// 8-bit floats).  New rows arrive as f16 / bf16; each value is divided by its pool's scale
// (float32, correctly rounded) and rounded to the nearest E4M3 code, saturating at 448.  Thread i
// turns 16 values (32 input bytes) of row i / (D / 16) of K and of V into one 16-code chunk of
// each pool row.
template <int SDT, int D>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(const uint8_t* __restrict__ k_new,
                                                            const uint8_t* __restrict__ v_new,
                                                            uint8_t* __restrict__ k_pool,
                                                            uint8_t* __restrict__ v_pool,
                                                            const int32_t* __restrict__ slots, int num_tokens,
                                                            int num_kv_heads, float k_scale, float v_scale) {
  constexpr int CPR = D / 16;        // 16-code chunks per pool row
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;   // the launch keeps every index below 2^31
  if (i >= (uint32_t)num_tokens * (uint32_t)num_kv_heads * CPR) return;
  const uint32_t c = i % CPR;
  const uint32_t row = i / CPR;
  const uint32_t t = row / (uint32_t)num_kv_heads, g = row % (uint32_t)num_kv_heads;
  // As in the 16-bit append: the rows' loads are issued before the slot is tested.
  const size_t src = (size_t)i * 32;
  u32x4 raw[4] = {__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_new + src)),
                  __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_new + src + 16)),
                  __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_new + src)),
                  __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_new + src + 16))};
  const int s = slots[t];
  asm volatile("" : "+v"(raw[0]), "+v"(raw[1]), "+v"(raw[2]), "+v"(raw[3]));
  if (s < 0) return;
  float kf[16], vf[16];
  unpack16<SDT>(raw[0], kf);
  unpack16<SDT>(raw[1], kf + 8);
  unpack16<SDT>(raw[2], vf);
  unpack16<SDT>(raw[3], vf + 8);
  u32x4 kc, vc;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t kw = pack_e4m3x2<false>(__fdiv_rn(kf[4 * w], k_scale), __fdiv_rn(kf[4 * w + 1], k_scale), 0u);
    kc[w] = pack_e4m3x2<true>(__fdiv_rn(kf[4 * w + 2], k_scale), __fdiv_rn(kf[4 * w + 3], k_scale), kw);
    const uint32_t vw = pack_e4m3x2<false>(__fdiv_rn(vf[4 * w], v_scale), __fdiv_rn(vf[4 * w + 1], v_scale), 0u);
    vc[w] = pack_e4m3x2<true>(__fdiv_rn(vf[4 * w + 2], v_scale), __fdiv_rn(vf[4 * w + 3], v_scale), vw);
  }
  const size_t dst = (((size_t)(s >> 4) * num_kv_heads + g) * 16 + (size_t)(s & 15)) * D + (size_t)c * 16;
  __builtin_nontemporal_store(kc, reinterpret_cast<u32x4*>(k_pool + dst));
  __builtin_nontemporal_store(vc, reinterpret_cast<u32x4*>(v_pool + dst));
}

template <int SDT, int D>
static hipError_t launch_append_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                    const int32_t* slots, int num_tokens, int num_kv_heads, float k_scale,
                                    float v_scale, hipStream_t stream) {
  const long long chunks = (long long)num_tokens * num_kv_heads * (D / 16);
  if (chunks + 255 > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)((chunks + 255) / 256));
  PK_LAUNCH((kv_append_fp8_kernel<SDT, D>), grid, dim3(256), stream, static_cast<const uint8_t*>(k_new),
            static_cast<const uint8_t*>(v_new), static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), slots,
            num_tokens, num_kv_heads, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_append_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                const int32_t* slots, int num_tokens, int num_kv_heads, int head_dim, int src_dtype,
                                float k_scale, float v_scale, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  if (src_dtype == kF16)
    return head_dim == 64 ? launch_append_fp8<kF16, 64>(k_new, v_new, k_pool, v_pool, slots, num_tokens, num_kv_heads,
                                                        k_scale, v_scale, stream)
                          : launch_append_fp8<kF16, 128>(k_new, v_new, k_pool, v_pool, slots, num_tokens,
                                                         num_kv_heads, k_scale, v_scale, stream);
  return head_dim == 64 ? launch_append_fp8<kBF16, 64>(k_new, v_new, k_pool, v_pool, slots, num_tokens, num_kv_heads,
                                                       k_scale, v_scale, stream)
                        : launch_append_fp8<kBF16, 128>(k_new, v_new, k_pool, v_pool, slots, num_tokens,
                                                        num_kv_heads, k_scale, v_scale, stream);
}

}  // namespace pk
