// KV append: slot-mapped copy of new K/V rows into the paged pools.
//
// A token's slot is physical_block * 16 + offset: the block the caller
// allocated for it ("LLM上下文缓存与状态复用机制的分析和探索", section 3.1:
// fixed-size blocks allocated on demand in non-contiguous memory).
//
// Pools: K [num_blocks][Hkv][16][D] (token rows), V [num_blocks][Hkv][D][16]
// (dim rows).  A run is a stretch of tokens whose slots follow each other
// inside one block (a request's new tokens fill its blocks in order, usually
// starting mid-block).  One workgroup serves one KV head and a window of 16
// consecutive tokens, and writes every run that starts inside the window, to
// its end (at most 15 tokens past the window).  So the 32-byte dim rows of a
// block that one run fills are written whole by one workgroup, instead of in
// two parts by two workgroups that may sit on different XCDs (a partly
// written sector costs a read-modify-write when it leaves the caches).
// K rows go straight to their slots with 16-byte stores; V rows are staged in
// LDS and each run leaves in the widest aligned stores its position allows.
#include "device_common.h"
#include "launch.h"

namespace pk {

// One element (EB bytes) read from LDS, zero-extended.
template <int EB>
__device__ __forceinline__ uint32_t lds_elem(const uint8_t* p) {
  if constexpr (EB == 4) return *reinterpret_cast<const uint32_t*>(p);
  else if constexpr (EB == 2) return *reinterpret_cast<const uint16_t*>(p);
  else return *p;
}

// Store u (a power of two, u * EB <= 16, dst aligned to u * EB) elements gathered from
// src, src + stride, ... with one store of u * EB bytes.
template <int EB>
__device__ __forceinline__ void store_elems(uint8_t* dst, const uint8_t* src, int stride, int u) {
  constexpr int MAXU = 16 / EB, PER = 4 / EB;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < MAXU; ++i)
    if (i < u) w[i / PER] |= lds_elem<EB>(src + i * stride) << (8 * EB * (i % PER));
  switch (u * EB) {
    case 16: *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]}; break;
    case 8: *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]}; break;
    case 4: *reinterpret_cast<uint32_t*>(dst) = w[0]; break;
    case 2: *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w[0]; break;
    default: *dst = (uint8_t)w[0]; break;
  }
}

// V rows staged in LDS (NT token rows of D elements of EB bytes; a negative slot is skipped) to
// the dim-major V tiles of their slots.  One thread per dim row walks the tokens run by run and
// writes each run with the widest aligned stores (16, 8, 4, 2 or 1 bytes), so a run that starts
// mid-block still leaves in wide stores.  (Sharing a dim row's runs among several threads
// measured slower.)
template <int EB, int D, int NT>
__device__ __forceinline__ void store_v_runs(const int* s_slot, const uint8_t* s_v, uint8_t* v_pool,
                                             int num_kv_heads, int g, int tid) {
  constexpr size_t TILE = (size_t)16 * D * EB;
  constexpr int ROW = D * EB;
  for (int d = tid; d < D; d += 256) {
    int t = 0;
    while (t < NT) {
      const int s = s_slot[t];
      if (s < 0) { ++t; continue; }
      int n = 1;
      while (t + n < NT && s_slot[t + n] == s + n && ((s + n) & 15) != 0) ++n;
      uint8_t* row = v_pool + ((size_t)(s >> 4) * num_kv_heads + g) * TILE + (size_t)d * 16 * EB;
      int p = s & 15;
      const int end = p + n;
      const uint8_t* src = s_v + t * ROW + d * EB;
      while (p < end) {
        int u = 16 / EB;
        while (u > 1 && ((p & (u - 1)) != 0 || p + u > end)) u >>= 1;
        store_elems<EB>(row + p * EB, src, ROW, u);
        src += u * ROW;
        p += u;
      }
      t += n;
    }
  }
}


template <int EB, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint8_t* __restrict__ k_new,
                                                        const uint8_t* __restrict__ v_new,
                                                        uint8_t* __restrict__ k_pool,
                                                        uint8_t* __restrict__ v_pool,
                                                        const int32_t* __restrict__ slots, int num_tokens,
                                                        int num_kv_heads) {
  constexpr int ROW = D * EB;        // bytes of one token's row for one head
  constexpr int CPR = ROW / 16;      // 16-byte chunks per row
  constexpr int NT = 32;             // tokens t0 .. t0 + 31: the window and the 15 tokens after it
  __shared__ int s_raw[NT + 1];      // slots of tokens t0 - 1 .. t0 + 31 (-1 outside the batch)
  __shared__ int s_slot[NT];         // slots of the tokens this workgroup writes, else -1
  __shared__ __attribute__((aligned(16))) uint8_t s_v[NT * ROW];

  const int t0 = blockIdx.x * 16;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < NT + 1) {
    const int i = t0 - 1 + tid;
    s_raw[tid] = (i >= 0 && i < num_tokens) ? slots[i] : -1;
  }
  __syncthreads();
  if (tid < NT) {
    // Token t0 + j continues its predecessor's run when its slot is the next one in the same
    // block.  It is ours when its run starts inside the window: for j < 16, unless every token
    // from t0 to it continues a run that began before t0; for j >= 16, when every token from
    // t0 + 16 to it continues (a run spans at most 16 tokens, so it then began at t0 + 1 or later).
    auto cont = [&](int j) {
      const int s = s_raw[j + 1], prev = s_raw[j];
      return s >= 0 && prev >= 0 && s == prev + 1 && (s & 15) != 0;
    };
    bool chain = true;
    for (int j = (tid < 16 ? 0 : 16); j <= tid; ++j) chain = chain && cont(j);
    const bool ours = tid < 16 ? !chain : chain;
    s_slot[tid] = ours ? s_raw[tid + 1] : -1;
  }
  __syncthreads();

  const size_t tile_bytes = (size_t)16 * ROW;
  for (int c = tid; c < NT * CPR; c += 256) {
    const int tok = c / CPR, wc = c % CPR;
    const int s = s_slot[tok];
    if (s >= 0) {
      const size_t src = ((size_t)(t0 + tok) * num_kv_heads + g) * ROW + (size_t)wc * 16;
      const u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + src);
      const size_t blk = (size_t)(s >> 4), off = (size_t)(s & 15);
      *reinterpret_cast<u32x4*>(k_pool + (blk * num_kv_heads + g) * tile_bytes + off * ROW + (size_t)wc * 16) = kv;
      *reinterpret_cast<u32x4*>(s_v + tok * ROW + wc * 16) = *reinterpret_cast<const u32x4*>(v_new + src);
    }
  }
  __syncthreads();

  store_v_runs<EB, D, NT>(s_slot, s_v, v_pool, num_kv_heads, g, tid);
}

template <int EB, int D>
static hipError_t launch_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                const int32_t* slots, int num_tokens, int num_kv_heads, hipStream_t stream) {
  dim3 grid((num_tokens + 15) / 16, num_kv_heads);
  PK_LAUNCH((kv_append_kernel<EB, D>), grid, dim3(256), stream,
                     static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new),
                     static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), slots, num_tokens,
                     num_kv_heads);
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
// (float32, correctly rounded) and rounded to the nearest E4M3 code, saturating at 448.  Same
// tiling as above: K rows go straight to their slots as 16-code chunks; V codes are staged in
// LDS and written as 4-byte runs of 4 consecutive tokens of one dim row where the slots allow
// (the pools' V tiles hold 16 one-byte tokens per dim row), else byte by byte.
template <int SDT, int D>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(const uint8_t* __restrict__ k_new,
                                                            const uint8_t* __restrict__ v_new,
                                                            uint8_t* __restrict__ k_pool,
                                                            uint8_t* __restrict__ v_pool,
                                                            const int32_t* __restrict__ slots, int num_tokens,
                                                            int num_kv_heads, float k_scale, float v_scale) {
  constexpr int IN_ROW = D * 2;      // bytes of one token's input row for one head
  constexpr int CPR = D / 16;        // 16-code chunks per token row
  __shared__ int s_slot[16];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[16 * D];

  const int t0 = blockIdx.x * 16;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < 16) s_slot[tid] = (t0 + tid < num_tokens) ? slots[t0 + tid] : -1;
  __syncthreads();

  const size_t tile_bytes = (size_t)16 * D;
  for (int c = tid; c < 16 * CPR; c += 256) {
    const int tok = c / CPR, wc = c % CPR;
    const int s = s_slot[tok];
    if (s < 0) continue;
    const size_t src = ((size_t)(t0 + tok) * num_kv_heads + g) * IN_ROW + (size_t)wc * 32;
    float kf[16], vf[16];
    unpack16<SDT>(*reinterpret_cast<const u32x4*>(k_new + src), kf);
    unpack16<SDT>(*reinterpret_cast<const u32x4*>(k_new + src + 16), kf + 8);
    unpack16<SDT>(*reinterpret_cast<const u32x4*>(v_new + src), vf);
    unpack16<SDT>(*reinterpret_cast<const u32x4*>(v_new + src + 16), vf + 8);
    u32x4 kc, vc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t kw = pack_e4m3x2<false>(__fdiv_rn(kf[4 * i], k_scale), __fdiv_rn(kf[4 * i + 1], k_scale), 0u);
      kc[i] = pack_e4m3x2<true>(__fdiv_rn(kf[4 * i + 2], k_scale), __fdiv_rn(kf[4 * i + 3], k_scale), kw);
      const uint32_t vw = pack_e4m3x2<false>(__fdiv_rn(vf[4 * i], v_scale), __fdiv_rn(vf[4 * i + 1], v_scale), 0u);
      vc[i] = pack_e4m3x2<true>(__fdiv_rn(vf[4 * i + 2], v_scale), __fdiv_rn(vf[4 * i + 3], v_scale), vw);
    }
    const size_t blk = (size_t)(s >> 4), off = (size_t)(s & 15);
    *reinterpret_cast<u32x4*>(k_pool + (blk * num_kv_heads + g) * tile_bytes + off * D + (size_t)wc * 16) = kc;
    *reinterpret_cast<u32x4*>(s_v + tok * D + wc * 16) = vc;
  }
  __syncthreads();

  for (int c = tid; c < D * 4; c += 256) {
    const int ts = (c % 4) * 4, d = c / 4;
    const int s0 = s_slot[ts];
    bool run = (s0 >= 0) && (s0 % 4) == 0;
#pragma unroll
    for (int e = 1; e < 4; ++e) run = run && (s_slot[ts + e] == s0 + e);
    if (run) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) word |= (uint32_t)s_v[(ts + e) * D + d] << (8 * e);
      const size_t blk = (size_t)(s0 >> 4), off = (size_t)(s0 & 15);
      *reinterpret_cast<uint32_t*>(v_pool + (blk * num_kv_heads + g) * tile_bytes + (size_t)d * 16 + off) = word;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = s_slot[ts + e];
        if (s < 0) continue;
        const size_t blk = (size_t)(s >> 4), off = (size_t)(s & 15);
        v_pool[(blk * num_kv_heads + g) * tile_bytes + (size_t)d * 16 + off] = s_v[(ts + e) * D + d];
      }
    }
  }
}

template <int SDT, int D>
static hipError_t launch_append_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                    const int32_t* slots, int num_tokens, int num_kv_heads, float k_scale,
                                    float v_scale, hipStream_t stream) {
  dim3 grid((num_tokens + 15) / 16, num_kv_heads);
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
