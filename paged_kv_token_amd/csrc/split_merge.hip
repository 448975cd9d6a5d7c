// Merge of split-KV partials into the attention output.
//
// "PersistentKV: Page-Aware Decode Scheduling for Long-Context LLM Serving on
// Commodity GPUs", section 2: a long context is cut into partitions handled
// in parallel and their results are merged.  For one (row, head) with
// partials (m_k, l_k, O_k): M = max m_k over partitions with l_k > 0,
// w_k = l_k exp(m_k - M), O = sum_k w_k O_k / sum_k w_k.
//
// One wave per (row, head): lanes read the P (m, l) pairs, reduce the max and
// the weight sum across the wave, park the weights in LDS, then stream the P
// partial rows of D fp32 values with 16-byte loads: D / 4 lanes cover one
// partition row (four dims each), so one pass reads 64 / (D / 4) partitions
// (two at D = 128, four at D = 64), and the lanes holding the same dims add
// their sums at the end (each partition's term is still one fma into one
// running sum per lane; the lanes' sums are added in a fixed order).
//
// Partials are laid out [row][head][P_stride]; with a row map, partial row c
// holds output row rowmap[2c] and only its first rowmap[2c + 1] partitions
// (the split-KV of pensieve_attn_fwd keeps only split requests' rows, each
// with its own partition count); without one, partial row c is output row c
// with P_stride partitions.
#include "device_common.h"
#include "launch.h"

namespace pk {

constexpr int kMaxMergePartitions = 256;

template <int DT, int D>
__global__ __launch_bounds__(256) void split_merge_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_m,
                                                          const float* __restrict__ part_l, int rows, int num_heads,
                                                          int P_stride, const int32_t* __restrict__ rowmap,
                                                          uint8_t* __restrict__ o) {
  __shared__ float s_w[4][kMaxMergePartitions];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int rh = blockIdx.x * 4 + wv;
  if (rh >= rows) return;  // whole wave leaves together; no block barrier follows
  const size_t base = (size_t)rh * P_stride;
  size_t out = rh;         // output (row, head) index
  int P = P_stride;
  if (rowmap) {
    const int c = rh / num_heads;
    out = (size_t)rowmap[2 * c] * num_heads + rh % num_heads;
    P = rowmap[2 * c + 1];
  }
  constexpr float kLog2e = 1.4426950408889634f;

  float M = -INFINITY;
  for (int p = lane; p < P; p += 64) {
    if (part_l[base + p] > 0.f) M = fmaxf(M, part_m[base + p]);
  }
  M = xor_max_from<1>(M);
  float W = 0.f;
  for (int p = lane; p < P; p += 64) {
    const float l = part_l[base + p];
    const float wgt = (l > 0.f) ? l * fast_exp2((part_m[base + p] - M) * kLog2e) : 0.f;
    s_w[wv][p] = wgt;
    W += wgt;
  }
  W = xor_sum_from<1>(W);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float inv = (W > 0.f) ? 1.f / W : 0.f;
  constexpr int LPR = D / 4;                // lanes per partition row
  constexpr int PPP = 64 / LPR;             // partitions per pass
  const int q4 = lane % LPR;                // dims 4 q4 .. 4 q4 + 3
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int p = lane / LPR; p < P; p += PPP) {
    const float wgt = s_w[wv][p];
    if (wgt != 0.f) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + (base + p) * D + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(wgt, v[e], acc[e]);
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < 4; ++e) store_elem<DT>(o, out * D + 4 * q4 + e, acc[e] * inv);
  }
}

template <int DT>
static hipError_t launch_merge_dt(const float* po, const float* pm, const float* pl, int rows, int num_heads,
                                  int head_dim, int P, const int32_t* rowmap, void* o, hipStream_t stream) {
  dim3 grid((rows + 3) / 4), block(256);
  if (head_dim == 64)
    PK_LAUNCH((split_merge_kernel<DT, 64>), grid, block, stream, po, pm, pl, rows, num_heads, P, rowmap,
                       (uint8_t*)o);
  else
    PK_LAUNCH((split_merge_kernel<DT, 128>), grid, block, stream, po, pm, pl, rows, num_heads, P, rowmap,
                       (uint8_t*)o);
  return hipGetLastError();
}

hipError_t launch_split_merge(const float* part_o, const float* part_m, const float* part_l, int rows, int num_heads,
                              int head_dim, int num_partitions, const int32_t* rowmap, int dtype, void* o,
                              hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  switch (dtype) {
    case kF32:
      return launch_merge_dt<kF32>(part_o, part_m, part_l, rows, num_heads, head_dim, num_partitions, rowmap, o, stream);
    case kF16:
      return launch_merge_dt<kF16>(part_o, part_m, part_l, rows, num_heads, head_dim, num_partitions, rowmap, o, stream);
    default:
      return launch_merge_dt<kBF16>(part_o, part_m, part_l, rows, num_heads, head_dim, num_partitions, rowmap, o,
                                    stream);
  }
}

}  // namespace pk
