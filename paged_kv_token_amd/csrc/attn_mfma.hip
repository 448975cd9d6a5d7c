// Matrix-core generalized paged attention (fp16 / bf16) for items with many
// query rows: prefill rows, recompute rows of partially evicted histories, and
// GQA groups ("Stateful Large Language Model Serving with Pensieve",
// Methodology: the kernel handles several input tokens over a cache that is
// scattered or partly dropped and recomputed).
//
// Work item: up to 128 query vectors = (128 / G) consecutive rows of one
// request x the G query heads sharing KV head g, over one partition of the
// request's KV blocks.  Four waves each own 32 query vectors (row-major over
// (token, head)).  KV is streamed in 64-token tiles (four 16-token blocks
// found through the block table): every thread loads its share of the tile
// into registers while the waves compute on the previous tile from LDS.
//
// Per wave and tile, with v_mfma_f32_32x32x16_{f16,bf16}:
//   S^T (64 keys x 32 rows)  = K_tile . Q^T        (2 x D/16 MFMAs)
//   online softmax on S^T in registers: each lane holds one query row's
//   scores, so the row max and sum stay in-lane except one exchange with
//   lane ^ 32
//   O^T (D x 32 rows)       += V^T_tile . P^T      (D/32 x 4 MFMAs)
// K rows are read from LDS in the order that swaps bits 2 and 3 of the MFMA
// row index; then the 8 scores a lane holds for a 16-key step are 8
// consecutive keys, which is exactly the layout of the P^T operand, and the
// V^T operand is one 16-byte LDS read of 8 consecutive keys of one dim row
// (the V pool stores each block as [D][16], so V^T needs no transpose).
#include "device_common.h"
#include "launch.h"

namespace pk {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int DT>
struct Mfma;

template <>
struct Mfma<kF16> {
  typedef _Float16 vec8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ _Float16 cvt(float x) { return (_Float16)x; }
};

template <>
struct Mfma<kBF16> {
  typedef __bf16 vec8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ __bf16 cvt(float x) { return (__bf16)x; }
};

__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = max(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = min(x, __shfl_xor(x, m, 64));
  return x;
}

// Zero the 16-bit elements e of an 8-element chunk whose key index first + e >= limit.
__device__ __forceinline__ u32x4 zero_keys_from(u32x4 v, int first, int limit) {
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    uint32_t keep = 0;
    if (first + 2 * wd < limit) keep |= 0x0000FFFFu;
    if (first + 2 * wd + 1 < limit) keep |= 0xFFFF0000u;
    v[wd] &= keep;
  }
  return v;
}

template <int DT, int D, int G>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(const AttnArgs a) {
  using MM = Mfma<DT>;
  using vec8 = typename MM::vec8;
  constexpr int KS = D / 16;           // k-steps of K.Q^T
  constexpr int MBD = D / 32;          // 32-dim blocks of O^T
  constexpr int KT = 64;               // keys per tile
  constexpr int TOKW = 32 / G;         // tokens per wave
  constexpr int KROW = D * 2 + 16;     // LDS bytes per K row (padded)
  constexpr int VROW = KT * 2 + 16;    // LDS bytes per V^T dim row (padded)
  constexpr int KBYTES = KT * KROW;
  constexpr int VBYTES = D * VROW;
  constexpr int OROW = D * 4 + 16;     // epilogue: fp32 output row
  constexpr int OBYTES = 128 * OROW;
  constexpr int LDS_BYTES = (KBYTES + VBYTES) > OBYTES ? (KBYTES + VBYTES) : OBYTES;
  constexpr int CB = 2 * D;            // 16-byte chunks per block tile
  constexpr int CPT = 4 * CB / 256;    // chunks per thread per tile (per tensor)
  constexpr int KCH = D / 8;           // 16-byte chunks per K row
  constexpr size_t TILE = (size_t)16 * D * 2;
  static_assert(G >= 1 && G <= 32 && (32 % G) == 0, "group size must divide 32");

  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ int s_wmax[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int h2 = lane >> 5;
  const int n = lane & 31;
  const WorkItem it = a.items[blockIdx.x];
  const int r = it.req, g = it.kv_head;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads;
  const int L = a.context_lens[r];
  const int row0 = a.cu_q_lens[r];
  const int q_r = a.cu_q_lens[r + 1] - row0;
  const float c = a.scale_log2;

  // ---- this lane's query row ----------------------------------------------------
  const int tok = w * TOKW + n / G;
  const bool row_valid = tok < it.q_count;
  const size_t qrow = (size_t)row0 + it.q_begin + (row_valid ? tok : 0);
  const int h = g * G + (n % G);
  int pos = -1;
  if (row_valid) pos = a.q_pos ? a.q_pos[qrow] : (L - q_r + it.q_begin + tok);

  vec8 qreg[KS];
  {
    const uint8_t* qp = a.q + (qrow * Hq + h) * (size_t)(D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(qp + (ks * 16 + 8 * h2) * 2));
  }
  const int pmax_w = uniform(wave_max_i(pos));
  const int pmin_w = uniform(wave_min_i(pos));
  if (lane == 0) s_wmax[w] = pmax_w;
  __syncthreads();
  const int pmax_wg = max(max(s_wmax[0], s_wmax[1]), max(s_wmax[2], s_wmax[3]));

  // ---- key range of this item ------------------------------------------------------
  const int nblk = (L + 15) >> 4;
  const int per = (nblk + it.num_parts - 1) / it.num_parts;
  const int kb0 = it.part * per;
  const int kb1 = min(kb0 + per, nblk);
  const int t_begin = kb0 * 16;
  const int t_valid = min(kb1 * 16, L);
  const int t_end = min(t_valid, pmax_wg + 1);
  const int ntiles = (t_end > t_begin) ? (t_end - t_begin + KT - 1) / KT : 0;

  const int32_t* bt = a.block_tables + (size_t)r * a.bt_stride;
  u32x4 kst[CPT], vst[CPT];
  auto load_tile = [&](int t0) {
    const int blk0 = t0 >> 4;
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int wbase = w * 64 + 256 * x;       // first chunk of this wave's load
      const int b = wbase / CB;                 // block within the tile (wave-uniform)
      const int ch = (wbase % CB) + lane;
      int lb = blk0 + b;
      lb = (lb < kb1) ? lb : kb0;               // past the partition: any block of it (masked)
      const size_t off = ((size_t)bt[lb] * Hkv + g) * TILE + (size_t)ch * 16;
      kst[x] = *reinterpret_cast<const u32x4*>(a.k_pool + off);
      vst[x] = *reinterpret_cast<const u32x4*>(a.v_pool + off);
    }
  };
  auto write_tile = [&](int t0) {
    const bool tail = t0 + KT > t_valid;
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      const int wbase = w * 64 + 256 * x;
      const int b = wbase / CB;
      const int ch = (wbase % CB) + lane;
      const int krow = b * 16 + ch / KCH, kcol = ch % KCH;
      const int vd = ch >> 1, vh = ch & 1;
      u32x4 kv = kst[x], vv = vst[x];
      if (tail) {
        if (t0 + krow >= t_valid) kv = u32x4{0, 0, 0, 0};
        vv = zero_keys_from(vv, t0 + b * 16 + vh * 8, t_valid);
      }
      *reinterpret_cast<u32x4*>(lds + krow * KROW + kcol * 16) = kv;
      *reinterpret_cast<u32x4*>(lds + KBYTES + vd * VROW + (b * 16 + vh * 8) * 2) = vv;
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[MBD];
#pragma unroll
  for (int j = 0; j < MBD; ++j) acc[j] = f32x16{};
  // LDS row of the K key that MFMA row (32 mb + n) multiplies: bits 2 and 3 swapped.
  const int krow_of_n = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);

  if (ntiles > 0) {
    load_tile(t_begin);
    write_tile(t_begin);
  }
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    const int t0 = t_begin + ti * KT;
    const bool more = ti + 1 < ntiles;
    if (more) load_tile(t0 + KT);
    if (t0 <= pmax_w) {
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
        const uint8_t* kp = lds + (32 * mb + krow_of_n) * KROW + h2 * 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const vec8 kop = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(kp + ks * 32));
          s[mb] = MM::mma(kop, qreg[ks], s[mb]);
        }
      }
      // s[mb][v] is the score of key t0 + 32 mb + 16 (v / 8) + 8 h2 + v % 8 for this lane's row.
      if ((t0 + KT - 1 > pmin_w) || (t0 + KT > t_valid)) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int tk = t0 + 32 * mb + 16 * (v >> 3) + 8 * h2 + (v & 7);
            s[mb][v] = (tk <= pos && tk < t_valid) ? s[mb][v] : -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[mb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float corr = fast_exp2((m_run - m_use) * c);
      const float mc = m_use * c;
      float ls = 0.f;
      vec8 pb[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(fmaf(s[mb][v], c, -mc));
          ls += p;
          pb[2 * mb + (v >> 3)][v & 7] = MM::cvt(p);
        }
      l_run = fmaf(l_run, corr, ls);
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < MBD; ++j) acc[j] *= corr;
#pragma unroll
      for (int j = 0; j < MBD; ++j) {
        const uint8_t* vp = lds + KBYTES + (32 * j + n) * VROW + h2 * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const vec8 vop = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(vp + ks * 32));
          acc[j] = MM::mma(vop, pb[ks], acc[j]);
        }
      }
    }
    __syncthreads();
    if (more) {
      write_tile(t0 + KT);
      __syncthreads();
    }
  }

  // ---- epilogue: normalise, stage rows in LDS, store coalesced -----------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  {
    uint8_t* orow = lds + (w * 32 + n) * OROW;
#pragma unroll
    for (int j = 0; j < MBD; ++j)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 val = {acc[j][4 * q4] * inv, acc[j][4 * q4 + 1] * inv, acc[j][4 * q4 + 2] * inv,
                     acc[j][4 * q4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + (32 * j + 8 * q4 + 4 * h2) * 4) = val;
      }
  }
  const bool split = a.write_partials || it.num_parts > 1;
  if (split && h2 == 0 && row_valid) {
    const size_t pi = (qrow * Hq + h) * a.part_stride + it.part;
    a.part_m[pi] = (m_run == -INFINITY) ? -INFINITY : m_run * a.scale;
    a.part_l[pi] = l_tot;
  }
  __syncthreads();
  if (!split) {
    constexpr int CHR = D / 8;   // 8-element output chunks per row
#pragma unroll
    for (int x = 0; x < 128 * CHR / 256; ++x) {
      const int ci = tid + 256 * x;
      const int rr = ci / CHR, cc = ci % CHR;
      const int otok = rr / G;
      if (otok >= it.q_count) continue;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(lds + rr * OROW + cc * 32);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(lds + rr * OROW + cc * 32 + 16);
      vec8 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) { ov[e] = MM::cvt(lo[e]); ov[4 + e] = MM::cvt(hi[e]); }
      const size_t orow_g = (size_t)row0 + it.q_begin + otok;
      const size_t dst = ((orow_g * Hq + g * G + (rr % G)) * D + cc * 8) * 2;
      *reinterpret_cast<u32x4*>(a.o + dst) = __builtin_bit_cast(u32x4, ov);
    }
  } else {
    constexpr int CHR = D / 4;   // 4-float chunks per row
#pragma unroll
    for (int x = 0; x < 128 * CHR / 256; ++x) {
      const int ci = tid + 256 * x;
      const int rr = ci / CHR, cc = ci % CHR;
      const int otok = rr / G;
      if (otok >= it.q_count) continue;
      const f32x4 val = *reinterpret_cast<const f32x4*>(lds + rr * OROW + cc * 16);
      const size_t orow_g = (size_t)row0 + it.q_begin + otok;
      const size_t pi = (orow_g * Hq + g * G + (rr % G)) * a.part_stride + it.part;
      *reinterpret_cast<f32x4*>(a.part_o + pi * D + cc * 4) = val;
    }
  }
}

template <int DT, int D>
static hipError_t launch_mfma_d(const AttnArgs& args, int group, hipStream_t stream) {
  dim3 grid(args.num_items), block(256);
  switch (group) {
    case 1: hipLaunchKernelGGL((attn_mfma_kernel<DT, D, 1>), grid, block, 0, stream, args); break;
    case 2: hipLaunchKernelGGL((attn_mfma_kernel<DT, D, 2>), grid, block, 0, stream, args); break;
    case 4: hipLaunchKernelGGL((attn_mfma_kernel<DT, D, 4>), grid, block, 0, stream, args); break;
    case 8: hipLaunchKernelGGL((attn_mfma_kernel<DT, D, 8>), grid, block, 0, stream, args); break;
    case 16: hipLaunchKernelGGL((attn_mfma_kernel<DT, D, 16>), grid, block, 0, stream, args); break;
    case 32: hipLaunchKernelGGL((attn_mfma_kernel<DT, D, 32>), grid, block, 0, stream, args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_mfma(const AttnArgs& args, int dtype, int head_dim, int group, hipStream_t stream) {
  if (args.num_items == 0) return hipSuccess;
  if (dtype == kF16)
    return head_dim == 64 ? launch_mfma_d<kF16, 64>(args, group, stream) : launch_mfma_d<kF16, 128>(args, group, stream);
  if (dtype == kBF16)
    return head_dim == 64 ? launch_mfma_d<kBF16, 64>(args, group, stream)
                          : launch_mfma_d<kBF16, 128>(args, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace pk
