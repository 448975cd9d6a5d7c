// Matrix-core generalized paged attention (fp16 / bf16) for items with many
// query rows: prefill rows, recompute rows of partially evicted histories, and
// GQA groups ("Stateful Large Language Model Serving with Pensieve",
// Methodology: the kernel handles several input tokens over a cache that is
// scattered or partly dropped and recomputed).
//
// Work item: up to 32 NW query vectors = (32 NW / G) consecutive rows of one
// request x the G query heads sharing KV head g, over one partition of the
// request's KV blocks.  NW = 4 or 8 waves each own 32 query vectors (row-major
// over (token, head)).  KV is streamed in 64-token tiles (four 16-token blocks
// found through the block table), each wave loading one block of every tile
// (with eight waves, half of one) straight into LDS one step ahead of its use,
// with one workgroup barrier per tile.  Four-wave workgroups run two to a CU;
// an eight-wave workgroup fills a CU alone (its epilogue needs 135 KB of LDS at
// d = 128) and feeds twice the query rows from each tile it loads.  Pools may hold f16 / bf16 or E4M3 codes (widened exactly on the way
// from LDS to the MFMA operands).
//
// Per wave and tile, with v_mfma_f32_32x32x16_{f16,bf16}:
//   S^T (64 keys x 32 rows)  = K_tile . Q^T        (2 x D/16 MFMAs)
//   online softmax on S^T in registers: each lane holds one query row's
//   scores, so the row max and sum stay in-lane except one exchange with
//   lane ^ 32
//   O^T (D x 32 rows)       += V^T_tile . P^T      (D/32 x 4 MFMAs)
// K rows are read from LDS in the order that swaps bits 2 and 3 of the MFMA
// row index; then the 8 scores a lane holds for a 16-key step are 8
// consecutive keys, which is exactly the layout of the P^T operand.  V tiles
// are token rows like K ([16][D] per block); each V^T operand (8 consecutive
// keys of one dim) comes from gfx950's transposing LDS reads:
// ds_read_b64_tr_b16 gives a lane one dim of 4 keys (two reads per operand),
// ds_read_b64_tr_b8 one dim of 8 E4M3 codes (one read per operand).
#include <climits>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pk {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int DT>
struct Mfma;

template <>
struct Mfma<kF16> {
  typedef _Float16 vec8 __attribute__((ext_vector_type(8)));
  // Eight E4M3 codes (bytes of w in order) as f16 values, exactly (two per conversion).
  static __device__ __forceinline__ vec8 from_e4m3(u32x2 w) {
    vec8 r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t word = w[i];
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true);
      r[4 * i] = lo[0]; r[4 * i + 1] = lo[1]; r[4 * i + 2] = hi[0]; r[4 * i + 3] = hi[1];
    }
    return r;
  }
  static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ _Float16 cvt(float x) { return (_Float16)x; }
  static __device__ __forceinline__ float dot2_ones(_Float16 a, _Float16 b, float acc) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 ab = {a, b}, one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(ab, one, acc, false);
  }
};

template <>
struct Mfma<kBF16> {
  typedef __bf16 vec8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ vec8 from_e4m3(u32x2 w) {
    vec8 r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t word = w[i];
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true);
      r[4 * i] = lo[0]; r[4 * i + 1] = lo[1]; r[4 * i + 2] = hi[0]; r[4 * i + 3] = hi[1];
    }
    return r;
  }
  static __device__ __forceinline__ f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ __bf16 cvt(float x) { return (__bf16)x; }
  static __device__ __forceinline__ float dot2_ones(__bf16 a, __bf16 b, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ab = {a, b}, one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(ab, one, acc, false);
  }
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

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): wait until at most N vector-memory operations are outstanding, or
// until every LDS / scalar-memory operation has finished.
template <int N>
constexpr int vmcnt_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}
constexpr int lgkmcnt0_imm() { return 63 | (3 << 14) | (7 << 4); }

// 16 bytes per lane from `base + voff` (a buffer resource of `nbytes` bytes: offsets past
// it read as zero) straight into LDS at `lds_dst + 16 * lane`.  Issued as inline assembly
// so that the compiler's wait-count tracking, which cannot tell one LDS stage from another,
// does not wait for these loads before every LDS read; callers wait for them explicitly
// with s_waitcnt vmcnt.  M0 carries the LDS address, bound as an input operand, so the
// compiler itself writes it and knows it holds that value.  NT: the non-temporal form, for
// K/V that no other workgroup of the launch reads.
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ void lds_dma16(const uint8_t* base, uint32_t nbytes, uint32_t voff, uint8_t* lds_dst) {
  const unsigned long long b = (unsigned long long)base;
  const i32x4 rsrc = {(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), (int)nbytes, kBufferWord3};
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(size_t)lds_dst);
  if constexpr (NT)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0) : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0) : "memory");
}

// Workgroup barrier that does not wait for outstanding memory operations (LDS-DMA
// loads of later tiles stay in flight); the wavefront-scope fences only keep the
// compiler from moving memory accesses across it.  Callers wait explicitly for
// what must be complete.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Max of x over lanes l and l ^ 32 (v_permlane32_swap moves the two halves past each other).
__device__ __forceinline__ float half_swap_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)pr[0]), __builtin_bit_cast(float, (int)pr[1]));
}

// XOR swizzle of the 16-byte chunk slots of V key row t in LDS: chunk c of row t lives in slot
// c ^ vswz(t).  The transposing reads of one V^T operand take 4 rows (2-byte elements) or 8
// rows (E4M3) of a few 16-byte chunks each; with these permutations the rows a half-wave (and
// each 16-lane group) reads fall in distinct banks, for 64 banks of 4 bytes with 32 lanes served
// per cycle as well as for 32 banks with 16 (derived by enumeration over every read).
template <int D, bool F8>
__device__ __forceinline__ int vswz_rows(int t) {
  if constexpr (!F8) return D == 128 ? 4 * (t & 3) + 2 * ((t >> 1) & 1) : 2 * (t & 3);   // 0,4,10,14 | 0,2,4,6
  else return D == 128 ? (t & 7) : ((t >> 1) & 3);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
// Transposing LDS reads (gfx950).  Within each group of 16 lanes: tr16 -- the 8-byte loads of
// lanes 4r .. 4r+3 form row r of a 4 x 16 matrix of 16-bit elements and lane i receives column
// i (row r's element in its element r); tr8 -- the loads of lanes 2r, 2r+1 form row r of an
// 8 x 16 byte matrix and lane i receives column i (row r's byte in its byte r).
__device__ __forceinline__ v4i16 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
}
__device__ __forceinline__ u32x2 lds_tr8(const uint8_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)p));
}

// XOR swizzle of the 16-byte chunk slots of K row r in LDS: chunk c of row r
// lives in slot c ^ kswz(r).  kswz swaps bits 2 and 3 of r (mod 16), the same
// permutation the MFMA row order uses, so the 8 or 16 lanes that read one
// chunk column from 8 or 16 different rows hit distinct bank groups.
template <int KCH>
__device__ __forceinline__ int kswz_rows(int r) {
  const int x = r & 15;
  return ((x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1)) & (KCH - 1);
}

// XOR swizzle of the 16-byte chunk slots of E4M3 K row t in LDS (rows of D bytes).  A K operand
// read takes one whole chunk per lane (two k-steps of 8 codes); the 16 rows a 16-lane group
// reads then fall in distinct banks, and so do the 8 rows of each 8-lane half (enumerated over
// every read for 64 banks with 16 lanes served per cycle and 32 banks with 8).
template <int D>
__device__ __forceinline__ int kswz8_rows(int t) {
  if constexpr (D == 128) return (t & 3) ^ ((t >> 2) & 1) ^ (((t >> 3) & 1) << 2);
  else return ((t >> 1) & 1) ^ ((t >> 2) & 1) ^ (((t >> 3) & 1) << 1);
}

template <int DT, int KVT, int D, int G, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_mfma_kernel(const AttnArgs a) {
  using MM = Mfma<DT>;
  using vec8 = typename MM::vec8;
  constexpr bool F8 = KVT == kFP8;        // pools hold E4M3 codes, widened to DT in registers
  constexpr int EB = F8 ? 1 : 2;          // bytes of a stored K / V element
  constexpr int KS = D / 16;              // k-steps of K.Q^T
  constexpr int MBD = D / 32;             // 32-dim blocks of O^T
  constexpr int KT = 64;                  // keys per tile (four blocks)
  constexpr int TOKW = 32 / G;            // tokens per wave
  constexpr int KROW = D * EB;            // bytes of one K row (one key)
  constexpr int BLK = 16 * KROW;          // bytes of one block's K (or V) tile
  constexpr int STAGE = 4 * BLK;          // one 64-key tile of K (or V)
  constexpr int NI = BLK / 1024;          // 1 KB LDS-DMA loads per block and tensor
  constexpr int KCH = KROW / 16;          // 16-byte chunks per K row
  constexpr int RPI = 1024 / KROW;        // K rows per DMA load
  static_assert(KVT == DT || F8, "stored K / V are the query type or E4M3 codes");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  constexpr int NT = 64 * NW;             // threads of the workgroup
  constexpr int NIW = NI * 4 / NW;        // 1 KB loads per wave, tensor and tile
  constexpr int OROW = D * 4 + 16;        // epilogue: fp32 output row
  constexpr int OBYTES = 32 * NW * OROW;
  constexpr int PIPE = 4 * STAGE;         // K stages 0,1 then V stages 0,1
  constexpr int LDS_BYTES = PIPE > OBYTES ? PIPE : OBYTES;
  static_assert(G >= 1 && G <= 32 && (32 % G) == 0, "group size must divide 32");
  static_assert(NIW >= 1 && NIW * NW == NI * 4, "a block tile must fill whole 1 KB loads of each wave");
  static_assert((KT * KCH) % NT == 0, "the tail zeroing covers whole tiles");

  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ int s_wmax[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int h2 = lane >> 5;
  const int n = lane & 31;
  const WorkItem it = a.items[blockIdx.x];
  if (it.q_count == 0) return;   // filler item (whole workgroup leaves before any barrier)
  const int r = it.req, g = it.kv_head;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads;
  const int L = a.context_lens[r];
  const int row0 = a.cu_q_lens[r];
  const int q_r = a.cu_q_lens[r + 1] - row0;
  const float c = a.scale_log2;
  constexpr float kSlack = 8.0f;          // log2 headroom before the running max must move
  const float slack_raw = kSlack / c;

  // ---- this lane's query row --------------------------------------------------------------
  // Row block of this wave, rotated by the workgroup index in four-wave workgroups: in items with
  // fewer than 128 query vectors the busy waves then fall on different SIMDs in the two
  // workgroups sharing a CU.
  const int wr = NW == 4 ? (w + (int)(blockIdx.x & 3)) & 3 : w;
  const int bw = w & 3;                   // block of each tile this wave loads
  const int jw = (w >> 2) * NIW;          // its first 1 KB load of that block
  const int tok = wr * TOKW + n / G;
  const bool row_valid = tok < it.q_count;
  const size_t qrow = (size_t)row0 + it.q_begin + (row_valid ? tok : 0);
  const int h = g * G + (n % G);
  int pos = -1;
  if (row_valid) pos = a.q_pos ? a.q_pos[qrow] : (L - q_r + it.q_begin + tok);

  // B operand of k-step ks: 8 query elements.  The 16 k-indices of a step may be any 16 dims as
  // long as the K operand uses the same: for 2-byte pools step ks takes dims 16 ks + 8 h2 .. + 7;
  // for E4M3 pools the steps come in pairs (2p, 2p + 1) whose lanes h2 take chunk 2p + h2 of the
  // K row (dims 16 (2p + h2) .. + 15) in one 16-byte read, 8 dims per step.
  vec8 qreg[KS];
  {
    const uint8_t* qp = a.q + (qrow * Hq + h) * (size_t)(D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int dim = F8 ? 16 * ((ks & ~1) + h2) + 8 * (ks & 1) : ks * 16 + 8 * h2;
      qreg[ks] = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(qp + dim * 2));
    }
  }
  const int pmax_w = uniform(wave_max_i(pos));
  const int pmin_w = uniform(wave_min_i(row_valid ? pos : INT_MAX));   // over valid rows only
  if (lane == 0) s_wmax[w] = pmax_w;
  __syncthreads();
  int pmax_wg = s_wmax[0];
#pragma unroll
  for (int x = 1; x < NW; ++x) pmax_wg = max(pmax_wg, s_wmax[x]);

  // ---- key range of this item ----------------------------------------------------------------
  const int nblk = (L + 15) >> 4;
  const int per = (nblk + it.num_parts - 1) / it.num_parts;
  const int kb0 = it.part * per;
  const int kb1 = min(kb0 + per, nblk);
  const int t_begin = kb0 * 16;
  const int t_valid = min(kb1 * 16, L);
  const int t_end = min(t_valid, pmax_wg + 1);
  const int ntiles = (t_end > t_begin) ? (t_end - t_begin + KT - 1) / KT : 0;

  // ---- LDS-DMA tile loads ---------------------------------------------------------------------
  // Wave w loads block w % 4 of each tile, K and V, with NIW buffer loads of 1 KB each straight
  // into LDS (lane l lands at +16 l): all NI loads of the block with four waves, loads
  // jw .. jw + NIW - 1 of them with eight.  K stage: row t (0..63) at t * KROW, chunk c in slot
  // c ^ kswz(t).  V stage: the same rows, chunk c in slot c ^ vswz(t).  Source offsets inside a
  // block tile depend only on the lane: computed once.
  uint32_t koff[NIW], voff[NIW];
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int t16 = (jw + j) * RPI + lane / KCH;
    const int ksw = F8 ? kswz8_rows<D>(t16) : kswz_rows<KCH>(t16);
    koff[j] = (uint32_t)(t16 * KROW + ((lane % KCH) ^ ksw) * 16);
    voff[j] = (uint32_t)(t16 * KROW + ((lane % KCH) ^ vswz_rows<D, F8>(t16)) * 16);
  }
  // Physical blocks this wave loads, held one per lane in a window of two VGPRs and read with
  // v_readlane, so that no scalar-load latency sits on the per-tile path: window k holds tiles
  // 64k .. 64k + 63 (lane l: tile 64k + l) in register k & 1.  Windows 0 and 1 are loaded
  // here; at tile 64k (k >= 1) the step refills the register of window k - 1, whose last block
  // was issued two steps earlier, with window k + 1, 62 steps before its first use.  Past the
  // partition any block of it serves (those keys are masked).
  const int32_t* const bt_row = a.block_tables + (size_t)r * a.bt_stride;
  auto window_block = [&](int k) {            // this lane's block of window k
    const int lb = kb0 + 4 * (64 * k + lane) + bw;
    return bt_row[lb < kb1 ? lb : kb0];
  };
  int btw0 = 0, btw1 = 0;
  if (kb0 < kb1) {
    btw0 = window_block(0);
    btw1 = window_block(1);
  }
  auto block_of = [&](int tile) {            // physical block loaded by this wave for `tile`
    return __builtin_amdgcn_readlane((tile & 64) ? btw1 : btw0, tile & 63);
  };
  // When the request's rows fit one item, no other item reads this KV head's tiles of the
  // partition and the loads are non-temporal; otherwise the items of the request's other rows
  // read the same tiles at about the same time, through L2.
  const bool read_once = uniform(q_r <= NW * TOKW ? 1 : 0) != 0;
  auto issue = [&](const uint8_t* pool, const uint32_t* offs, int tile, uint8_t* stage) {
    const uint8_t* src = pool + ((size_t)block_of(tile) * Hkv + g) * BLK;
    if (read_once) {
#pragma unroll
      for (int j = 0; j < NIW; ++j) lds_dma16<true>(src, BLK, offs[j], stage + bw * BLK + (jw + j) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < NIW; ++j) lds_dma16<false>(src, BLK, offs[j], stage + bw * BLK + (jw + j) * 1024);
    }
  };
  auto kstage = [&](int tile) { return lds + (tile & 1) * STAGE; };
  auto vstage = [&](int tile) { return lds + (2 + (tile & 1)) * STAGE; };

  float m_run = -INFINITY, l_run = 0.f;
  float m_top = -INFINITY;                   // true running max (m_run may lag it by up to the slack)
  f32x16 acc[MBD];
#pragma unroll
  for (int j = 0; j < MBD; ++j) acc[j] = f32x16{};
  // LDS row of the K key that MFMA row (32 mb + n) multiplies: bits 2 and 3 swapped.
  const int krow_of_n = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);

  // Per-lane LDS read offsets, fixed for the whole item.  K: the elements of row
  // (32 mb + krow_of_n) for k-step ks live at krd[ks] + 32 KROW mb inside a K stage (2-byte
  // elements: chunk 2 ks + h2; E4M3: chunk ks + h2 for even ks, read whole for steps ks, ks + 1).  V: lane n + 32 h2 needs
  // dim 32 j + n of keys 16 ks + 8 h2 .. + 7 (block ks of the tile).  In its 16-lane group
  // (gm = bit 4 of the lane: dims 16 gm .. 16 gm + 15 of the 32) the transposing read points
  // the lane at key row 8 h2 + rr (+ 4 for the second read of 2-byte elements) of block ks, at
  // the 8 bytes that hold dims 32 j + 16 gm + 4 c4 .. + 3 (2-byte; rr = bits 2..3, c4 = bits
  // 0..1 of the lane) or 32 j + 16 gm + 8 hb .. + 7 (E4M3; rr = bits 1..3, hb = bit 0); the
  // row's swizzle depends only on rr.  vrd[j] is that address for block 0 and the first read.
  uint32_t krd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if constexpr (F8)
      krd[ks] = (uint32_t)(krow_of_n * KROW + ((((ks & ~1) + h2) ^ kswz8_rows<D>(krow_of_n)) * 16));
    else
      krd[ks] = (uint32_t)(krow_of_n * KROW + (((2 * ks + h2) ^ kswz_rows<KCH>(krow_of_n)) * 16));
  }
  uint32_t vrd[MBD];
  {
    const int gm = (lane >> 4) & 1;
    const int rr = F8 ? (lane & 15) >> 1 : (lane & 15) >> 2;
    const int sw = vswz_rows<D, F8>(rr);
#pragma unroll
    for (int j = 0; j < MBD; ++j) {
      if constexpr (F8) {
        vrd[j] = (uint32_t)((8 * h2 + rr) * KROW + (((2 * j) | gm) ^ sw) * 16 + (lane & 1) * 8);
      } else {
        const int c4 = lane & 3;
        vrd[j] = (uint32_t)((8 * h2 + rr) * KROW + (((4 * j) | (2 * gm) | (c4 >> 1)) ^ sw) * 16 + (c4 & 1) * 8);
      }
    }
  }
  // V^T operand of k-step ks (block ks of the tile), dims 32 j .. 32 j + 31.
  auto v_operand = [&](const uint8_t* vst, int j, int ks) -> vec8 {
    const uint8_t* p = vst + vrd[j] + ks * BLK;
    if constexpr (F8) {
      return MM::from_e4m3(lds_tr8(p));
    } else {
      const v4i16 lo = lds_tr16(p), hi = lds_tr16(p + 4 * KROW);
      const v4i16 both[2] = {lo, hi};
      return __builtin_bit_cast(vec8, both);
    }
  };
  // One 8-element K operand of 2-byte elements from LDS (E4M3 rows are read two steps at a time
  // and widened exactly in qk below).
  auto operand = [&](const uint8_t* p) -> vec8 { return __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(p)); };

  // S^T of one tile for this lane's row: s[mb][v] is key t0 + 32 mb + 16 (v / 8) + 8 h2 + v % 8.
  // K operands are read in batches of four k-steps for both 32-key halves, and the two
  // independent accumulator chains alternate, so LDS latency overlaps the MFMAs.
  constexpr int KPRE_STEPS = 3;              // k-steps of K operands read before the row max
  auto qk = [&](const uint8_t* ks_base, f32x16* sc, const vec8 (*kfirst)[2]) {
    sc[0] = f32x16{};
    sc[1] = f32x16{};
#pragma unroll
    for (int k0 = 0; k0 < KS; k0 += 4) {
      vec8 kop[4][2];
      if (kfirst && k0 == 0) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            kop[kk][mb] = kk < KPRE_STEPS ? kfirst[kk][mb] : operand(ks_base + krd[kk] + mb * 32 * KROW);
      } else if constexpr (F8) {
#pragma unroll
        for (int kk = 0; kk < 4; kk += 2)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const u32x4 w16 = *reinterpret_cast<const u32x4*>(ks_base + krd[k0 + kk] + mb * 32 * KROW);
            kop[kk][mb] = MM::from_e4m3(u32x2{w16[0], w16[1]});
            kop[kk + 1][mb] = MM::from_e4m3(u32x2{w16[2], w16[3]});
          }
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            kop[kk][mb] = operand(ks_base + krd[k0 + kk] + mb * 32 * KROW);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sc[mb] = MM::mma(kop[kk][mb], qreg[k0 + kk], sc[mb]);
    }
  };

  f32x16 s_cur[2], s_nxt[2];
  // A wave whose 32 query vectors all lie past the item's rows (short prefill items) still
  // loads its share of every tile and meets every barrier, but computes nothing.
  const bool wave_idle = uniform(wr * TOKW >= it.q_count ? 1 : 0) != 0;
  wait_vmem_all();                           // query rows and positions have landed
  if (ntiles > 0) {
    issue(a.k_pool, koff, 0, kstage(0));
    if (ntiles > 1) issue(a.k_pool, koff, 1, kstage(1));
    issue(a.v_pool, voff, 0, vstage(0));
    if (ntiles > 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * NIW>());
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm<NIW>());
    lds_barrier();
    if (!wave_idle) qk(lds, s_cur, nullptr);
  }

  // One tile: PAR is ti & 1 (the K stage of tile ti + 1 and the V stage of tile ti are
  // compile-time offsets); s_cur holds S^T of tile ti, s_nxt receives S^T of tile ti + 1.
  auto tile_step = [&](int ti, auto par, f32x16* s_cur, f32x16* s_nxt) {
    constexpr int PAR = decltype(par)::value;
    uint8_t* const k_next = lds + (1 - PAR) * STAGE;     // K stage of tile ti + 1
    uint8_t* const k_free = lds + PAR * STAGE;           // K stage of tile ti (free after QK(ti))
    uint8_t* const v_cur = lds + (2 + PAR) * STAGE;      // V stage of tile ti
    uint8_t* const v_free = lds + (3 - PAR) * STAGE;     // V stage of tile ti - 1
    const int t0 = t_begin + ti * KT;
    const bool k2 = ti + 2 < ntiles, v1 = ti + 1 < ntiles;
    // The only loads in flight are this wave's K(ti + 1) and V(ti), issued one step ago: wait for
    // them; then one barrier makes every wave's loads visible and frees the stages of K(ti) (QK(ti)
    // is done) and V(ti - 1) (PV(ti - 1) is done) for the next loads.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    lds_barrier();
    if (k2) issue(a.k_pool, koff, ti + 2, k_free);
    if (v1) issue(a.v_pool, voff, ti + 1, v_free);
    if (PAR == 0 && ti >= 64 && (ti & 63) == 0 && ti + 64 < ntiles) {
      // Refill: window ti / 64 + 1 into the register of window ti / 64 - 1 (same parity).
      const int nxt = window_block((ti >> 6) + 1);
      if (ti & 64) btw0 = nxt;
      else btw1 = nxt;
    }
    if (t0 + KT > t_valid) {
      // Tail: keys at or past t_valid must contribute exactly 0; stale V may hold NaN, so their
      // whole rows are zeroed in LDS.
#pragma unroll
      for (int x = 0; x < KT * KCH / NT; ++x) {
        const int ci = tid + NT * x;         // (key row, chunk) pairs of the tile
        const int row = ci / KCH, ch = ci % KCH;
        if (t0 + row >= t_valid) *reinterpret_cast<u32x4*>(v_cur + row * KROW + ch * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
      lds_barrier();
    }
    if (wave_idle) return;                    // loads and barriers only
    // 2-byte pools at d = 128: the K operands of the first KPRE_STEPS k-steps of the next tile's
    // QK are read here, before the row max below, so that their LDS latency overlaps it (the next
    // tile's scores are not live yet, so their registers are free).
    constexpr bool KPRE = !F8 && D == 128;
    vec8 kfirst[4][2] = {};
    if constexpr (KPRE) {
#pragma unroll
      for (int kk = 0; kk < KPRE_STEPS; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) kfirst[kk][mb] = operand(k_next + krd[kk] + mb * 32 * KROW);
    }
    // Masking (diagonal and tail tiles only): key offset 32 mb + 16 (v / 8) + v % 8 from
    // t0 + 8 h2 is visible iff it is <= lim.
    if ((t0 + KT - 1 > pmin_w) || (t0 + KT > t_valid)) {
      const int lim = min(pos, t_valid - 1) - (t0 + 8 * h2);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          s_cur[mb][v] = (32 * mb + 16 * (v >> 3) + (v & 7) <= lim) ? s_cur[mb][v] : -INFINITY;
    }
    // Row max over the 32 scores of this lane, then with the lane holding the other 32 keys.
    float mx = fmaxf(s_cur[0][0], s_cur[0][1]);
#pragma unroll
    for (int v = 2; v < 16; v += 2) mx = fmaxf(fmaxf(mx, s_cur[0][v]), s_cur[0][v + 1]);
#pragma unroll
    for (int v = 0; v < 16; v += 2) mx = fmaxf(fmaxf(mx, s_cur[1][v]), s_cur[1][v + 1]);
    mx = half_swap_max(mx);
    m_top = fmaxf(m_top, mx);
    // The running max moves only when some row's tile max exceeds it by more than
    // kSlack / c (raw score units); otherwise weights stay <= 2^kSlack and the
    // accumulator needs no rescale.  Any row's growth moves all rows of the wave.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + slack_raw) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = fast_exp2((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c);
      l_run *= corr;
#pragma unroll
      for (int j = 0; j < MBD; ++j) acc[j] *= corr;
      m_run = m_new;
    }
    // One straight-line region: QK of the next tile (independent MFMAs), the weights of
    // this tile (VALU), then O^T += V^T P^T.  The next tile's QK is computed even when it
    // does not exist (its result is then never read), so that no branch splits the region
    // and the scheduler can interleave the MFMAs with the exponentials.
    qk(k_next, s_nxt, KPRE ? kfirst : nullptr);
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
    vec8 pb[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) pb[2 * mb + (v >> 3)][v & 7] = MM::cvt(fast_exp2(fmaf(s_cur[mb][v], c, -mc)));
    // Row sum of the rounded weights (the same values the P.V product uses).
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2) l_run = MM::dot2_ones(pb[ks][e], pb[ks][e + 1], l_run);
    // O^T += V^T P^T: k-step ks is block ks of the tile.
#pragma unroll
    for (int j0 = 0; j0 < MBD; j0 += 2) {
      vec8 vop[2][4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          vop[jj][ks] = v_operand(v_cur, j0 + jj, ks);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[j0 + jj] = MM::mma(vop[jj][ks], pb[ks], acc[j0 + jj]);
    }
    // Issue order for the region above: each MFMA followed by three VALU instructions, so the
    // exponentials of this tile run while the QK MFMAs of the next one execute, and the weight
    // conversions and row sums while the PV MFMAs do.  Left to itself the scheduler issues the QK
    // MFMAs back to back, each behind its own LDS operand reads.  At D = 128 the LDS operand
    // reads are also placed: six K reads were issued before the row max (their latency overlaps
    // it; 1 % on the GQA recompute batch), two more go out before the first QK MFMA and the rest
    // one after each MFMA; twelve transposing V reads (six V^T operands) go out before the first
    // PV MFMA and two after each, so every MFMA finds its operand loaded several MFMAs earlier
    // (253-256 VGPRs, no spills; 2-3 % on the long-context and GQA recompute batches; eight and
    // sixteen reads ahead spill, and so do eight K reads before the row max at G = 8), and the
    // QK phase takes two VALU instructions per MFMA (1 % on the long-context batch).  E4M3 tiles
    // keep the scheduler's order: their operand widening adds four VALU conversions per MFMA,
    // and the same pattern made them slower.
    constexpr int VA = 12;                   // V reads issued ahead of the first PV MFMA
    if constexpr (!F8 && D == 128) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);      // LDS reads
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {                       // QK of the next tile
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
        if (i < 2 * KS - 2 * KPRE_STEPS - 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);     // two VALU instructions
      }
      __builtin_amdgcn_sched_group_barrier(0x100, VA, 0);
#pragma unroll
      for (int i = 0; i < 4 * MBD; ++i) {                      // PV of this tile
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (2 * i < 8 * MBD - VA) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    } else if constexpr (!F8) {
#pragma unroll
      for (int i = 0; i < 2 * KS + 4 * MBD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // three VALU instructions
      }
    }
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  for (int ti = 0; ti < ntiles; ti += 2) {
    tile_step(ti, P0{}, s_cur, s_nxt);
    if (ti + 1 < ntiles) tile_step(ti + 1, P1{}, s_nxt, s_cur);
  }

  // ---- epilogue: normalise, stage rows in LDS, store coalesced -----------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if constexpr (F8) inv *= a.v_scale;
  __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
  __syncthreads();                            // every wave is done reading the pipeline stages
  {
    uint8_t* orow = lds + (wr * 32 + n) * OROW;
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
  // Partial row of the item's first query row (partials of split requests may be compacted).
  const size_t prow0 = (a.part_row_base ? (size_t)a.part_row_base[r] : (size_t)row0) + it.q_begin;
  if (split && h2 == 0 && row_valid) {
    // Report l relative to the true max: l_top = l_tot * exp2((m_run - m_top) c).
    const size_t pi = ((prow0 + tok) * Hq + h) * a.part_stride + it.part;
    const bool any = m_top != -INFINITY;
    a.part_m[pi] = any ? m_top * a.scale : -INFINITY;
    a.part_l[pi] = any ? l_tot * fast_exp2((m_run - m_top) * c) : 0.f;
  }
  __syncthreads();
  if (!split) {
    constexpr int CHR = D / 8;   // 8-element output chunks per row
#pragma unroll
    for (int x = 0; x < 32 * NW * CHR / NT; ++x) {
      const int ci = tid + NT * x;
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
    for (int x = 0; x < 32 * NW * CHR / NT; ++x) {
      const int ci = tid + NT * x;
      const int rr = ci / CHR, cc = ci % CHR;
      const int otok = rr / G;
      if (otok >= it.q_count) continue;
      const f32x4 val = *reinterpret_cast<const f32x4*>(lds + rr * OROW + cc * 16);
      const size_t pi = ((prow0 + otok) * Hq + g * G + (rr % G)) * a.part_stride + it.part;
      *reinterpret_cast<f32x4*>(a.part_o + pi * D + cc * 4) = val;
    }
  }
}

template <int DT, int KVT, int D, int NW>
static hipError_t launch_mfma_d(const AttnArgs& args, int group, hipStream_t stream) {
  dim3 grid(args.num_items), block(64 * NW);
  switch (group) {
    case 1: PK_LAUNCH((attn_mfma_kernel<DT, KVT, D, 1, NW>), grid, block, stream, args); break;
    case 2: PK_LAUNCH((attn_mfma_kernel<DT, KVT, D, 2, NW>), grid, block, stream, args); break;
    case 4: PK_LAUNCH((attn_mfma_kernel<DT, KVT, D, 4, NW>), grid, block, stream, args); break;
    case 8: PK_LAUNCH((attn_mfma_kernel<DT, KVT, D, 8, NW>), grid, block, stream, args); break;
    case 16: PK_LAUNCH((attn_mfma_kernel<DT, KVT, D, 16, NW>), grid, block, stream, args); break;
    case 32: PK_LAUNCH((attn_mfma_kernel<DT, KVT, D, 32, NW>), grid, block, stream, args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Eight-wave workgroups exist for 2-byte pools and for E4M3 pools at d = 128 (an E4M3 block
// tile at d = 64 is a single 1 KB load, which two waves cannot share).
template <int DT, int KVT>
static hipError_t launch_mfma_dt(const AttnArgs& args, int head_dim, int group, bool wide, hipStream_t stream) {
  if constexpr (KVT == kFP8) {
    if (wide) return head_dim == 128 ? launch_mfma_d<DT, KVT, 128, 8>(args, group, stream) : hipErrorInvalidValue;
  } else {
    if (wide)
      return head_dim == 64 ? launch_mfma_d<DT, KVT, 64, 8>(args, group, stream)
                            : launch_mfma_d<DT, KVT, 128, 8>(args, group, stream);
  }
  return head_dim == 64 ? launch_mfma_d<DT, KVT, 64, 4>(args, group, stream)
                        : launch_mfma_d<DT, KVT, 128, 4>(args, group, stream);
}

hipError_t launch_attn_mfma(const AttnArgs& args, int dtype, int kv_dtype, int head_dim, int group, bool wide,
                            hipStream_t stream) {
  if (args.num_items == 0) return hipSuccess;
  const bool f8 = kv_dtype == kFP8;
  if (dtype == kF16) return f8 ? launch_mfma_dt<kF16, kFP8>(args, head_dim, group, wide, stream)
                               : launch_mfma_dt<kF16, kF16>(args, head_dim, group, wide, stream);
  if (dtype == kBF16) return f8 ? launch_mfma_dt<kBF16, kFP8>(args, head_dim, group, wide, stream)
                                : launch_mfma_dt<kBF16, kBF16>(args, head_dim, group, wide, stream);
  return hipErrorInvalidValue;
}

}  // namespace pk
