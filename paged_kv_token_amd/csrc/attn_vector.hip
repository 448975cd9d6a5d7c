// Vector-ALU generalized paged attention for items with few query vectors.
//
// Serves decode rows (one new token), small groups of rows, and every fp32
// batch.  One workgroup (4 waves) handles one work item: up to NQ query
// vectors (tokens x query heads of one KV head) of one request, over one
// partition of that request's KV blocks.  The four waves stride over the
// item's blocks, each with two blocks' loads in flight; each wave keeps an
// online softmax per query vector in registers and the waves merge through
// LDS at the end.
//
// Per 16-token block a wave issues 16-byte loads that cover the K tile and the
// V tile (both [16][D], token rows) exactly once (64 lanes x 16 B per load), so
// HBM traffic is the algorithmic K/V bytes.  Lane l of load i holds dims
// (l % LPT) * EPC .. +EPC of token i * TPI + l / LPT, of K and of V alike; the
// q.k partial sums are reduced over the LPT lanes of a token with DPP row
// operations, which leaves every one of those lanes holding the token's score,
// so each lane weights its own V elements with no exchange between lanes.  The
// lanes holding the same dims of different tokens are summed once per item.
//
// Semantics ("Stateful Large Language Model Serving with Pensieve", Abstract:
// attention of several new tokens over a non-contiguous cache): row i sees
// keys at positions 0..pos(i) of its request; masked keys and slots past the
// context length never enter the sums (scores are selected to -inf and V
// elements past the context length are selected to 0, so stale NaN cannot
// leak in).
#include "device_common.h"
#include "launch.h"

namespace pk {

// 16 E4M3 codes widened exactly to 8 packed pairs of the query type.
template <int DT>
__device__ __forceinline__ void widen_e4m3x16(const u32x4 w, uint32_t* pairs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word = w[i];
    if constexpr (DT == kF16) {
      pairs[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false));
      pairs[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true));
    } else {
      pairs[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false));
      pairs[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true));
    }
  }
}

// acc + a.x * b.x + a.y * b.y over packed pairs of the query type, in fp32.
template <int DT>
__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float acc) {
  if constexpr (DT == kF16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), acc, false);
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), acc, false);
  }
}

template <int DT, int KT, int D, int NQ>
__global__ __launch_bounds__(256) void attn_vector_kernel(const AttnArgs a) {
  constexpr int EQ = DTypeInfo<DT>::bytes;   // bytes of a Q / O element
  constexpr int EB = DTypeInfo<KT>::bytes;   // bytes of a stored K / V element
  constexpr int EPC = 16 / EB;          // K / V elements per 16-byte chunk
  constexpr int QCH = EPC * EQ / 16;    // 16-byte Q chunks matching one K chunk
  constexpr int LPT = D * EB / 16;      // lanes holding one K token row
  constexpr int TPI = 64 / LPT;         // K tokens per load
  constexpr int KI = 16 / TPI;          // K loads (and V loads) per block
  constexpr int NW = 4;
  constexpr size_t TILE = (size_t)16 * D * EB;
  static_assert(KT == DT || KT == kFP8, "stored K / V are the query type or E4M3 codes");
  static_assert(LPT >= 1 && LPT <= 32, "unsupported row width");

  __shared__ float s_m[NW][NQ];
  __shared__ float s_l[NW][NQ];
  __shared__ float s_acc[NW][NQ][D];

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const WorkItem it = a.items[blockIdx.x];
  const int r = it.req, g = it.kv_head;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int L = a.context_lens[r];
  const int row0 = a.cu_q_lens[r];
  const int q_r = a.cu_q_lens[r + 1] - row0;
  const int hc = it.head_count;
  const int nrows = it.q_count * hc;
  const float c = a.scale_log2;

  // ---- query vectors and their positions -----------------------------------
  // fp32 pools: the lane's query elements as floats.  f16 / bf16 and E4M3 pools: kept packed
  // (two elements per register) and multiplied with the stored (or widened) K pairs by
  // two-element dot products with fp32 accumulation; the products of two 16-bit floats are
  // exact in fp32.
  constexpr bool F8 = KT == kFP8;
  constexpr bool PK = KT != kF32;       // packed query pairs
  float qv[NQ][PK ? 1 : EPC];
  uint32_t qh[NQ][PK ? EPC / 2 : 1];
  int qpos[NQ];
  int pmin = 0x7fffffff, pmax = -1;
  const int dim0 = (lane % LPT) * EPC;
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    const bool valid = n < nrows;
    const int tok = valid ? n / hc : 0;
    const int h = g * G + it.head_begin + (valid ? n % hc : 0);
    const int row = row0 + it.q_begin + tok;
#pragma unroll
    for (int qc = 0; qc < QCH; ++qc) {
      const u32x4 qw = *reinterpret_cast<const u32x4*>(a.q + (((size_t)row * Hq + h) * D + dim0) * EQ + qc * 16);
      if constexpr (PK) {
#pragma unroll
        for (int e = 0; e < 4; ++e) qh[n][4 * qc + e] = qw[e];
      } else {
        unpack16<DT>(qw, qv[n] + qc * (16 / EQ));
      }
    }
    int p = -1;
    if (valid) p = a.q_pos ? a.q_pos[row] : (L - q_r + it.q_begin + tok);
    qpos[n] = p;
    if (valid) { pmin = min(pmin, p); pmax = max(pmax, p); }
  }

  // ---- this item's block range ----------------------------------------------
  const int nblk = (L + 15) >> 4;
  const int per = (nblk + it.num_parts - 1) / it.num_parts;
  const int kb0 = it.part * per;
  const int kb1 = min(min(kb0 + per, nblk), (pmax >> 4) + 1);

  float m[NQ], l[NQ], acc[NQ][EPC];     // acc: this lane's dims dim0 .. dim0 + EPC - 1
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    m[n] = -INFINITY; l[n] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[n][e] = 0.f;
  }

  const const_i32_ptr bt = as_const(a.block_tables) + (size_t)r * a.bt_stride;
  // An item holding every row and query head of its request and KV head is the only reader of
  // its K/V: those loads are non-temporal.
  const bool read_once = uniform(hc == G && it.q_count == q_r ? 1 : 0) != 0;
  auto load = [&](int blk, u32x4* kr, u32x4* vr) {
    const int phys = bt[uniform(blk)];
    const uint8_t* kt = a.k_pool + ((size_t)phys * Hkv + g) * TILE;
    const uint8_t* vt = a.v_pool + ((size_t)phys * Hkv + g) * TILE;
    if (read_once) {
#pragma unroll
      for (int i = 0; i < KI; ++i) kr[i] = tile_load16<true>(kt, (uint32_t)TILE, (uint32_t)(i * 64 + lane) * 16u);
#pragma unroll
      for (int i = 0; i < KI; ++i) vr[i] = tile_load16<true>(vt, (uint32_t)TILE, (uint32_t)(i * 64 + lane) * 16u);
    } else {
#pragma unroll
      for (int i = 0; i < KI; ++i) kr[i] = tile_load16(kt, (uint32_t)TILE, (uint32_t)(i * 64 + lane) * 16u);
#pragma unroll
      for (int i = 0; i < KI; ++i) vr[i] = tile_load16(vt, (uint32_t)TILE, (uint32_t)(i * 64 + lane) * 16u);
    }
  };

  auto process = [&](int blk, const u32x4* kr, const u32x4* vr) {
    const int base = blk * 16;
    const bool need_mask = base + 15 > pmin;
    float sc[NQ][KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      if constexpr (F8) {
        uint32_t kp[EPC / 2];
        widen_e4m3x16<DT>(kr[i], kp);
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < EPC / 2; ++e) s = dot2_acc<DT>(qh[n][e], kp[e], s);
          sc[n][i] = group_sum<LPT>(s);
        }
      } else if constexpr (PK) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < EPC / 2; ++e) s = dot2_acc<DT>(qh[n][e], kr[i][e], s);
          sc[n][i] = group_sum<LPT>(s);
        }
      } else {
        float kf[EPC];
        unpack16<KT>(kr[i], kf);
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < EPC; ++e) s = fmaf(qv[n][e], kf[e], s);
          sc[n][i] = group_sum<LPT>(s);
        }
      }
    }
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int t = base + i * TPI + lane / LPT;
#pragma unroll
        for (int n = 0; n < NQ; ++n) sc[n][i] = (t <= qpos[n]) ? sc[n][i] : -INFINITY;
      }
    }
    // V elements of this lane's tokens; keys at or past the context length must contribute
    // exactly 0 (stale slots may hold NaN), so they are selected to 0, not multiplied by 0.
    const bool zero_tail = base + 16 > L;
    float vf[KI][EPC];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      unpack16<KT>(vr[i], vf[i]);
      if (zero_tail && base + i * TPI + lane / LPT >= L) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) vf[i][e] = 0.f;
      }
    }
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      float bm = sc[n][0];
#pragma unroll
      for (int i = 1; i < KI; ++i) bm = fmaxf(bm, sc[n][i]);
      bm = xor_max_from<LPT>(bm);
      const float m_new = fmaxf(m[n], bm);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float corr = fast_exp2((m[n] - m_use) * c);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[n][e] *= corr;
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const float p = fast_exp2((sc[n][i] - m_use) * c);
        ps += p;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[n][e] = fmaf(p, vf[i][e], acc[n][e]);
      }
      l[n] = l[n] * corr + ps;
      m[n] = m_new;
    }
  };

  {
    // Two blocks in flight per wave: three register sets rotate by unrolling, and the loads
    // of block b + 2 NW are issued before block b is processed.  Loads past the item's last
    // block fetch that block again (unused, and still in L2), so every step issues the same
    // loads and the compiler's wait counts stay exact.
    u32x4 ka[KI], va[KI], kb[KI], vb[KI], kc[KI], vc[KI];
    const int b0 = kb0 + w;
    auto clamp_blk = [&](int b) { return b < kb1 ? b : kb1 - 1; };
    wait_vmem_all();
    if (b0 < kb1) {
      load(b0, ka, va);
      load(clamp_blk(b0 + NW), kb, vb);
      for (int blk = b0; blk < kb1; blk += 3 * NW) {
        load(clamp_blk(blk + 2 * NW), kc, vc);
        process(blk, ka, va);
        if (blk + NW >= kb1) break;
        load(clamp_blk(blk + 3 * NW), ka, va);
        process(blk + NW, kb, vb);
        if (blk + 2 * NW >= kb1) break;
        load(clamp_blk(blk + 4 * NW), kb, vb);
        process(blk + 2 * NW, kc, vc);
      }
      wait_vmem_all();     // the unused loads of the last step have landed
    }
  }

  // ---- merge the waves --------------------------------------------------------
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    const float lt = xor_sum_from<LPT>(l[n]);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float v = xor_sum_from<LPT>(acc[n][e]);     // over the lanes holding the same dims
      if (lane < LPT) s_acc[w][n][dim0 + e] = v;
    }
    if (lane == 0) { s_m[w][n] = m[n]; s_l[w][n] = lt; }
  }
  __syncthreads();

  const bool split = a.write_partials || it.num_parts > 1;
  // Partial row of the item's first query row (partials of split requests may be compacted).
  const size_t prow0 = (a.part_row_base ? (size_t)a.part_row_base[r] : (size_t)row0) + it.q_begin;
  for (int idx = threadIdx.x; idx < nrows * D; idx += 256) {
    const int n = idx / D, d = idx % D;
    float M = s_m[0][n];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, s_m[ww][n]);
    float lsum = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float f = fast_exp2((s_m[ww][n] - M) * c);
        lsum += f * s_l[ww][n];
        o += f * s_acc[ww][n][d];
      }
      o /= lsum;
      if constexpr (KT == kFP8) o *= a.v_scale;
    }
    const int tok = n / hc;
    const int h = g * G + it.head_begin + n % hc;
    const size_t row = (size_t)row0 + it.q_begin + tok;
    if (!split) {
      store_elem<DT>(a.o, (row * Hq + h) * D + d, o);
    } else {
      const size_t pi = ((prow0 + tok) * Hq + h) * a.part_stride + it.part;
      a.part_o[pi * D + d] = o;
      if (d == 0) {
        a.part_m[pi] = (M == -INFINITY) ? -INFINITY : M * a.scale;
        a.part_l[pi] = lsum;
      }
    }
  }
}

template <int DT, int KT, int D>
static hipError_t launch_vec_d(const AttnArgs& args, int rows, hipStream_t stream) {
  dim3 grid(args.num_items), block(256);
  switch (rows) {
    case 1: PK_LAUNCH((attn_vector_kernel<DT, KT, D, 1>), grid, block, stream, args); break;
    case 2: PK_LAUNCH((attn_vector_kernel<DT, KT, D, 2>), grid, block, stream, args); break;
    case 4: PK_LAUNCH((attn_vector_kernel<DT, KT, D, 4>), grid, block, stream, args); break;
    default: PK_LAUNCH((attn_vector_kernel<DT, KT, D, 8>), grid, block, stream, args); break;
  }
  return hipGetLastError();
}

template <int DT, int KT>
static hipError_t launch_vec_dt(const AttnArgs& args, int head_dim, int rows, hipStream_t stream) {
  return head_dim == 64 ? launch_vec_d<DT, KT, 64>(args, rows, stream) : launch_vec_d<DT, KT, 128>(args, rows, stream);
}

hipError_t launch_attn_vector(const AttnArgs& args, int dtype, int kv_dtype, int head_dim, int rows_per_item,
                              hipStream_t stream) {
  if (args.num_items == 0) return hipSuccess;
  if (kv_dtype == kFP8) {
    return dtype == kF16 ? launch_vec_dt<kF16, kFP8>(args, head_dim, rows_per_item, stream)
                         : launch_vec_dt<kBF16, kFP8>(args, head_dim, rows_per_item, stream);
  }
  switch (dtype) {
    case kF32: return launch_vec_dt<kF32, kF32>(args, head_dim, rows_per_item, stream);
    case kF16: return launch_vec_dt<kF16, kF16>(args, head_dim, rows_per_item, stream);
    default: return launch_vec_dt<kBF16, kBF16>(args, head_dim, rows_per_item, stream);
  }
}

}  // namespace pk
