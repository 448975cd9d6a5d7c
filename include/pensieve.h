/*
 * pensieve.h -- C ABI of libpensieve: generalized paged attention for gfx950.
 *
 * The operation: in a unified batch of requests, every new query row of a
 * request attends to that request's cached conversation K/V plus, causally,
 * to the request's own new rows.  The K/V lives in fixed-size blocks of a
 * shared pool, found through a per-request block table, so one request's KV
 * is spread over non-contiguous memory ("Stateful Large Language Model
 * Serving with Pensieve", Abstract and Methodology: the PagedAttention kernel
 * generalised to several input tokens over a non-contiguous GPU cache;
 * "LLM上下文缓存与状态复用机制的分析和探索", section 3.1: fixed-size blocks
 * allocated on demand in non-contiguous memory).  Prefill requests, decode
 * requests (one new row) and recompute rows (history tokens whose cache was
 * dropped, recomputed ahead of the new rows -- Pensieve, Methodology) all run
 * in one call.  Long contexts may be split into partitions whose partial
 * results are merged ("PersistentKV: Page-Aware Decode Scheduling for
 * Long-Context LLM Serving on Commodity GPUs", section 2, the split strategy).
 *
 * Conventions shared by every call
 * --------------------------------
 * - All data pointers are DEVICE pointers unless the name ends in _host.
 *   The caller allocates and owns every buffer; the library keeps no pointer
 *   after a call returns.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   device work is enqueued on it asynchronously; a call returns before the
 *   GPU finishes.  Host arrays (_host) are fully read before the call returns.
 * - Element type of Q, O and both pools: pensieve_dtype (F32, F16, BF16);
 *   with F16/BF16 queries the pools may instead hold FP8_E4M3 codes
 *   (desc.kv_dtype, with a scale per pool).
 *   Arithmetic: dot products, softmax and accumulation in fp32; on F16/BF16
 *   the softmax weights are rounded to the input type before the P.V product;
 *   outputs are rounded to nearest-even.  E4M3 codes are widened exactly
 *   (every E4M3 value is an F16 and a BF16 value); the K scale is folded into
 *   the softmax scale and the V scale into the output normalisation.
 * - block_size must be 16; head_dim must be 64 or 128; num_heads must be a
 *   multiple of num_kv_heads.  Query head h reads KV head
 *   h / (num_heads / num_kv_heads).
 * - Layouts (row-major):
 *     q, o          [total_q][num_heads][head_dim]; rows of request r are
 *                   cu_q_lens[r] .. cu_q_lens[r+1]-1
 *     k_pool        [num_blocks][num_kv_heads][16][head_dim]   (token rows)
 *     v_pool        [num_blocks][num_kv_heads][16][head_dim]   (token rows)
 *     block_tables  [num_reqs][block_table_stride] int32: logical block j
 *                   of request r lives in physical block block_tables[r][j]
 *   Position t of request r is stored at offset t % 16 of physical block
 *   block_tables[r][t / 16]; its slot is that block * 16 + t % 16.
 * - context_lens[r] counts every KV position of request r resident after the
 *   append of this step (history + recomputed + new).  A row at position p
 *   sees keys 0..p.  Slots at positions >= context_lens[r], unused blocks and
 *   block-table entries past ceil(context_lens[r]/16) may hold any bits, NaN
 *   included; the output does not depend on them and they are never read.
 * - Library-owned resources.  The library allocates no device memory on
 *   the calls' paths (callers pass workspace), but keeps three kinds of
 *   process-wide state, created on first use per device and held until the
 *   process ends: (1) a ring of 32 page-locked, device-mapped host slots
 *   (one 16 MiB slab, a slot grown alone past 512 KiB, and an 8 KiB
 *   page-locked flag array through which the copy kernel reports that it
 *   has read a slot) through which pensieve_attn_fwd,
 *   pensieve_attn_split_partial and the swaps upload their host-built work
 *   lists with a small copy kernel on `stream`;
 *   (2) a non-blocking side stream with two events: when a plan mixes
 *   matrix-core and vector items and the matrix-core items alone cannot
 *   fill the GPU, the vector items run on it, forked from and joined back
 *   into `stream` with events (PENSIEVE_FLAG_SINGLE_STREAM keeps every
 *   launch on `stream`); (3) the device scratch array of
 *   pensieve_attn_fwd_noalloc (64 MiB per GPU, allocated with the code
 *   object).  Because work lists are built and uploaded at every call, the
 *   calls refuse a stream that is being captured into a graph
 *   (UNSUPPORTED).
 * - Errors: every call returns a status.  Problems visible on the host
 *   (null pointers, bad sizes, inconsistent host lengths, too small a
 *   workspace) return INVALID_ARG / UNSUPPORTED / WORKSPACE_TOO_SMALL before
 *   anything is enqueued.  A failed HIP call returns ERR_HIP.
 *   pensieve_last_error() then describes the failure (per thread).
 *   The contents of device arrays are the caller's contract: slots and block
 *   ids in range, no duplicate slot in one append, query positions strictly
 *   increasing within a request and below its context length, device length
 *   arrays equal to their host copies.  With PENSIEVE_DEBUG=1 in the
 *   environment (read at every call), pensieve_kv_append(_fp8) and the
 *   attention calls first copy those device arrays to the host (waiting for
 *   `stream`) and return INVALID_ARG on a violation before anything of the
 *   call is enqueued; they never read the pools to do so.  Debugging and
 *   tests only: it synchronises every call.
 *   A call that finds its staging slot ((1) above) still being read by an
 *   earlier copy waits for it up to PENSIEVE_STAGE_WAIT_US microseconds
 *   (default 2 000 000, read at each such wait), then synchronises the
 *   device once; a slot still unreported after that is an ERR_HIP failure.
 */
#ifndef PENSIEVE_H
#define PENSIEVE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pensieve_status {
  PENSIEVE_OK = 0,
  PENSIEVE_ERR_INVALID_ARG = 1,
  PENSIEVE_ERR_UNSUPPORTED = 2,
  PENSIEVE_ERR_WORKSPACE_TOO_SMALL = 3,
  PENSIEVE_ERR_HIP = 4
} pensieve_status;

/* PENSIEVE_FP8_E4M3: pool storage only -- OCP 8-bit floats E4M3 (sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN,
 * largest finite 448), each pool with one float32 scale: the value read back is
 * the decoded code times the pool's scale ("LLM上下文缓存与状态复用机制的分析和探索",
 * section 4(3): the KV cache stored in FP8 to halve its memory). */
typedef enum pensieve_dtype {
  PENSIEVE_F32 = 0,
  PENSIEVE_F16 = 1,
  PENSIEVE_BF16 = 2,
  PENSIEVE_FP8_E4M3 = 3
} pensieve_dtype;

/* pensieve_batch_desc.flags: route every work item to the vector-ALU kernel
 * (on F16/BF16 the matrix-core kernel otherwise serves requests with more
 * than 8 query vectors (rows x heads per KV head) and every request of head
 * groups of 4 or more).  Results agree within the stated tolerances either
 * way. */
#define PENSIEVE_FLAG_VECTOR_ONLY 1
/* pensieve_batch_desc.flags: pensieve_attn_fwd keeps every request whole (no
 * adaptive split-KV; no partials, no merge). */
#define PENSIEVE_FLAG_NO_SPLIT 2
/* pensieve_batch_desc.flags: every launch of the call stays on the caller's
 * stream (no fork of vector items onto the library's side stream).  Results
 * are identical either way. */
#define PENSIEVE_FLAG_SINGLE_STREAM 4

/* Shape of one unified batch plus host copies of its lengths (used to
 * validate and to plan the work; the device copies passed to the compute
 * calls must hold the same values). */
typedef struct pensieve_batch_desc {
  int32_t num_reqs;
  int32_t num_heads;            /* query heads Hq */
  int32_t num_kv_heads;         /* KV heads Hkv; divides Hq */
  int32_t head_dim;             /* 64 or 128 */
  int32_t block_size;           /* 16 */
  int32_t num_blocks;           /* blocks in each pool */
  int32_t block_table_stride;   /* int32 entries per block-table row */
  int32_t dtype;                /* pensieve_dtype of Q and O (F32, F16, BF16) */
  float softmax_scale;          /* scale on q.k before the softmax, e.g. 1/sqrt(head_dim); > 0 */
  int32_t flags;                /* 0, or PENSIEVE_FLAG_VECTOR_ONLY | PENSIEVE_FLAG_NO_SPLIT */
  const int32_t* context_lens_host;  /* [num_reqs] */
  const int32_t* cu_q_lens_host;     /* [num_reqs + 1], cu_q_lens_host[0] == 0 */
  int32_t kv_dtype;             /* element type of both pools: dtype itself, or
                                   PENSIEVE_FP8_E4M3 when dtype is F16 or BF16 */
  float k_scale, v_scale;       /* FP8_E4M3 pools: value = code * scale (finite, > 0);
                                   ignored for other pools */
  const int32_t* q_pos_host;    /* [total_q] host copy of the q_pos array passed to the
                                   attention calls, or NULL.  Read only to plan: each
                                   matrix-core work item is costed by the keys its rows can
                                   see, and the items are spread over the XCDs by that cost.
                                   When NULL while q_pos is given, an item is costed by its
                                   request's whole context.  It never changes a result; values
                                   that differ from q_pos only change the work balance. */
} pensieve_batch_desc;

/* Library version string, e.g. "pensieve 0.1 gfx950". */
const char* pensieve_version(void);

/* Text of the last failure on the calling thread ("" after success). */
const char* pensieve_last_error(void);

/*
 * KV append: for every token t in [0, num_tokens) with slot_mapping[t] >= 0,
 * write k_new[t] into k_pool at block slot/16, offset slot%16 (a [Hkv][d]
 * row set) and v_new[t] into v_pool at the same place.  A negative slot
 * skips the token.  The copy is
 * bit-exact; nothing else in the pools changes.
 *   k_new, v_new  [num_tokens][num_kv_heads][head_dim], dtype elements
 *   slot_mapping  [num_tokens] int32, each < num_blocks*16, no duplicates
 * Follows the block-pool contract of the blog post cited above (section
 * 3.1): new tokens land in whatever block the caller allocated.
 */
pensieve_status pensieve_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                   const int32_t* slot_mapping, int32_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t num_blocks, int32_t dtype, void* stream);

/*
 * KV append into FP8_E4M3 pools: as pensieve_kv_append, but k_new / v_new hold
 * src_dtype (F16 or BF16) values and each pool element receives the E4M3 code
 * of value / scale (k_scale for K, v_scale for V): the quotient is computed in
 * float32 with correct rounding, magnitudes beyond 448 saturate to +-448, and
 * the rest round to the nearest code, ties to even; NaN stays NaN.  The pools
 * are [num_blocks][Hkv][16][d] bytes each.  Scales
 * must be finite and > 0 (INVALID_ARG otherwise).  Reading: the pages name
 * FP8 KV storage without a format or a scaling rule; OCP E4M3 with one scale
 * per pool is taken ("LLM上下文缓存与状态复用机制的分析和探索", section 4(3)).
 */
pensieve_status pensieve_kv_append_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                       const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t src_dtype,
                                       float k_scale, float v_scale, void* stream);

/*
 * Block swap with a host tier ("Stateful Large Language Model Serving with
 * Pensieve", Methodology and AI Executive Summary: cached KV tokens move
 * between a GPU tier and a CPU tier, swapped ahead of time with transfers
 * pipelined behind computation).  The host tier k_host/v_host has the pools'
 * block layout ([num_host_blocks][Hkv][16][d] each)
 * and must be page-locked host memory mapped for the device (hipHostMalloc,
 * or a pinned torch tensor).  A swap copies n whole blocks, every KV head:
 *   pensieve_kv_swap_out: host block host_blocks[i] = device block device_blocks[i]
 *   pensieve_kv_swap_in:  device block device_blocks[i] = host block host_blocks[i]
 * The block lists are host arrays of n int32, read before the call returns;
 * every id must lie in its pool and destinations must be distinct
 * (INVALID_ARG otherwise, before anything is enqueued).  The copy is
 * bit-exact and asynchronous on `stream`: run a swap-in on a second stream
 * beside the current step's attention, and make the step that reads the
 * blocks wait for it (an event).  Nothing else in either tier changes.
 */
pensieve_status pensieve_kv_swap_out(void* k_pool, void* v_pool, int32_t num_blocks, void* k_host,
                                     void* v_host, int32_t num_host_blocks,
                                     const int32_t* device_blocks_host, const int32_t* host_blocks_host,
                                     int32_t n, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                     void* stream);
pensieve_status pensieve_kv_swap_in(void* k_pool, void* v_pool, int32_t num_blocks, void* k_host,
                                    void* v_host, int32_t num_host_blocks,
                                    const int32_t* host_blocks_host, const int32_t* device_blocks_host,
                                    int32_t n, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                    void* stream);

/*
 * Cache planning for one serving step (host only: no device work, no stream).
 * "Stateful Large Language Model Serving with Pensieve", Methodology: cached
 * KV is dropped block by block, weighing a conversation's activity against
 * the cost of recomputing what is dropped, and dropped tokens are recomputed
 * with the conversation's next turn.
 *
 * A conversation is described by pensieve_conversation:
 *   cached_tokens   positions 0..cached_tokens-1 were computed earlier; their
 *                   KV sits in logical blocks 0..ceil(cached_tokens/16)-1
 *   dropped_blocks  leading logical blocks 0..dropped_blocks-1 no longer hold
 *                   KV on the device (their physical blocks were given back);
 *                   at most ceil(cached_tokens/16)
 *   new_tokens      tokens this step brings (0: not scheduled this step)
 *   activity        weight >= 0 of keeping the conversation's cache (e.g. the
 *                   inverse of its idle time); how it is measured is the
 *                   caller's policy
 */
typedef struct pensieve_conversation {
  int32_t cached_tokens;
  int32_t dropped_blocks;
  int32_t new_tokens;
  float activity;
} pensieve_conversation;

/*
 * Choose which blocks to drop so that the step fits in free_blocks.  The step
 * takes, per scheduled conversation, dropped_blocks fresh blocks for its
 * recomputed leading blocks plus the logical blocks its new tokens open.
 * When that exceeds free_blocks, blocks of UNSCHEDULED conversations are
 * dropped one at a time, leading resident block first, always the one of
 * least cost activity * (j + 1) for logical block j (a block's recompute cost
 * grows with the context it attends over; ties go to the lower conversation
 * index) -- the least-cost set of that many leading-first drops.
 * evict_blocks_host[c] receives how many more leading blocks conversation c
 * drops (its logical blocks dropped_blocks .. dropped_blocks+evict-1; the
 * caller frees them and adds evict to dropped_blocks); *freed_blocks their
 * sum.  UNSUPPORTED when even dropping every unscheduled block is not enough
 * (the outputs then hold that maximal drop).
 */
pensieve_status pensieve_cache_plan_evictions(const pensieve_conversation* conversations, int32_t n,
                                              int32_t free_blocks, int32_t* evict_blocks_host,
                                              int32_t* freed_blocks);

/*
 * Build the unified batch of one step from the scheduled conversations
 * (new_tokens > 0), in conversation order: request r serves conversation
 * request_conv_host[r].  Its query rows are the recompute rows -- every
 * position of its dropped blocks, 0 .. min(16*dropped_blocks, cached_tokens)-1
 * -- followed by its new rows cached_tokens .. cached_tokens+new_tokens-1;
 * q_pos_host gives each row's position (strictly increasing in a request),
 * context_lens_host[r] = cached_tokens + new_tokens.  Fresh physical blocks
 * are taken from free_list_host in order: first for the dropped logical blocks
 * 0..dropped_blocks-1, then for the logical blocks the new tokens open.
 * block_tables_host [n][block_table_stride] (conversation rows) is updated in
 * place with them and copied, per request, into req_block_tables_host
 * [num_reqs][block_table_stride]; slot_mapping_host gives each row's append
 * slot (feed it to pensieve_kv_append with the rows' recomputed and new K/V,
 * and q_pos_host, cu_q_lens_host, context_lens_host and req_block_tables_host
 * to pensieve_attn_fwd).  After the step the caller sets cached_tokens +=
 * new_tokens and dropped_blocks = 0.
 *   *num_reqs, *total_rows, *blocks_used   sizes of the batch (always written)
 *   max_rows < 0: sizes only, no other output is touched; otherwise the row
 *   arrays hold max_rows entries, cu_q_lens_host num_reqs+1, request_conv_host
 *   and context_lens_host num_reqs.
 * INVALID_ARG on inconsistent conversations, a block_table_stride too small
 * for a scheduled conversation, too few rows or free blocks, before any
 * output array is written.
 */
pensieve_status pensieve_cache_build_batch(const pensieve_conversation* conversations, int32_t n,
                                           int32_t* block_tables_host, int32_t block_table_stride,
                                           const int32_t* free_list_host, int32_t free_count, int32_t max_rows,
                                           int32_t* num_reqs, int32_t* total_rows, int32_t* blocks_used,
                                           int32_t* request_conv_host, int32_t* cu_q_lens_host,
                                           int32_t* context_lens_host, int32_t* q_pos_host,
                                           int32_t* slot_mapping_host, int32_t* req_block_tables_host);

/*
 * Workspace needed by pensieve_attn_fwd (num_partitions == 0) or by
 * pensieve_attn_split_partial (num_partitions >= 1) for this batch.  The
 * workspace holds the device copy of the work list and, when
 * pensieve_attn_fwd splits long requests, their fp32 partial results
 * (about rows x Hq x P x (head_dim + 2) x 4 bytes for the split requests'
 * rows only); it is plain device memory owned by the caller, needs no
 * initialisation and may be reused by the next call on the same stream.
 * The size depends on every field of the descriptor (q_pos_host included:
 * it changes how the work list is laid out), so size the workspace with the
 * descriptor the attention call receives.
 */
pensieve_status pensieve_attn_workspace_size(const pensieve_batch_desc* desc, int32_t num_partitions,
                                             size_t* bytes);

/*
 * Generalized paged attention (Pensieve, Abstract/Methodology):
 *   o[i][h][:] = sum_t softmax_t(scale * q[i][h].K[t]) V[t],  t <= pos(i),
 * over the KV of row i's request, head h / (Hq/Hkv).
 *   q_pos  [total_q] int32 absolute position of every row, or NULL: row j of
 *          request r (0-based) then sits at context_lens[r] - q_r + j.
 * o must not alias q.  Run the pensieve_kv_append of this step's rows first,
 * on the same stream.
 * A request whose work items would run much longer than the batch's fair
 * share (total KV blocks over all items / 512, at least 64 blocks) is cut
 * into P partitions of its blocks (split-KV, as in the PersistentKV paper,
 * section 2); its partials go to the workspace and a final merge kernel
 * combines them into o.  Short batches are never split, and no request is
 * when desc->flags has PENSIEVE_FLAG_NO_SPLIT.
 */
pensieve_status pensieve_attn_fwd(const pensieve_batch_desc* desc, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* cu_q_lens,
                                  const int32_t* q_pos, void* o, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * pensieve_attn_fwd without a workspace, for callers that cannot allocate
 * device memory (code that may not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics and kernels
 * as pensieve_attn_fwd, and bitwise the same output; the work list and the
 * split partials live in a library-owned device array of 64 MiB per GPU
 * instead of a caller workspace.  The call allocates nothing (no hipMalloc,
 * hipHostMalloc, stream or event creation): it runs every launch on
 * `stream` (as with PENSIEVE_FLAG_SINGLE_STREAM) and copies the work list
 * from pageable host memory with hipMemcpyAsync, which may wait for earlier
 * work on `stream` before it returns.  A batch whose work list and partials
 * exceed 64 MiB returns WORKSPACE_TOO_SMALL (pensieve_attn_workspace_size
 * reports the bytes it would need).  Every call on one GPU shares that GPU's
 * array: calls on one stream are ordered, but calls that may overlap on one
 * GPU (several streams or host threads) race and must not be issued.  A
 * stream being captured into a graph is refused (UNSUPPORTED).
 */
pensieve_status pensieve_attn_fwd_noalloc(const pensieve_batch_desc* desc, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_tables,
                                          const int32_t* context_lens, const int32_t* cu_q_lens,
                                          const int32_t* q_pos, void* o, void* stream);

/*
 * Split-KV partials (PersistentKV, section 2: one long context cut into
 * partitions processed in parallel).  Request r's logical blocks are cut
 * into num_partitions ranges of S = ceil(ceil(L_r/16)/num_partitions)
 * blocks: partition k covers positions [16kS, 16(k+1)S) clipped to [0, L_r).
 * For row i, head h, partition k (index (i*Hq + h)*P + k):
 *   part_m[.] = max scaled score over the visible keys of the partition
 *   part_l[.] = sum of exp(score - part_m) over them
 *   part_o[.][:] = that weighted sum of V divided by part_l (fp32)
 * A partition with no visible key stores m = -inf, l = 0, o = 0.
 *   part_o [total_q][Hq][P][head_dim] fp32, part_m/part_l [total_q][Hq][P] fp32
 */
pensieve_status pensieve_attn_split_partial(const pensieve_batch_desc* desc, int32_t num_partitions,
                                            const void* q, const void* k_pool, const void* v_pool,
                                            const int32_t* block_tables, const int32_t* context_lens,
                                            const int32_t* cu_q_lens, const int32_t* q_pos,
                                            float* part_o, float* part_m, float* part_l,
                                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Merge of split partials: M = max_k m_k, w_k = l_k exp(m_k - M),
 * o = sum_k w_k o_k / sum_k w_k (partitions with l_k = 0 weigh nothing),
 * rounded to dtype.  Shapes as in pensieve_attn_split_partial; o is
 * [total_q][num_heads][head_dim].
 */
pensieve_status pensieve_attn_split_merge(const float* part_o, const float* part_m, const float* part_l,
                                          int32_t total_q, int32_t num_heads, int32_t head_dim,
                                          int32_t num_partitions, int32_t dtype, void* o, void* stream);

/*
 * Host-only introspection of the work list pensieve_attn_fwd
 * (num_partitions == 0) or pensieve_attn_split_partial would build for this
 * batch.  Writes up to max_items records of 10 int32 each:
 *   {kernel, request, kv_head, first row in request, rows, partition,
 *    partitions, estimated cost, first query head of the group, heads}
 * with kernel 0 = vector path, 1 = matrix-core path, in launch order, and
 * sets *num_items to the full count.  No GPU is touched.  A matrix-core
 * item holds up to 128 query vectors (rows x heads), or up to 256 in calls
 * whose four-wave items would not fill one round of the GPU (about 512
 * items) and that hold a request of more than 128 query vectors per KV
 * head, with 2-byte pools or E4M3 pools at head_dim 128: those run in
 * eight-wave workgroups.
 */
pensieve_status pensieve_debug_plan(const pensieve_batch_desc* desc, int32_t num_partitions,
                                    int32_t* items_host, int32_t max_items, int32_t* num_items);

/*
 * Per-launch timing trace.  While enabled, every kernel the library
 * launches records start and stop events through its own dispatch packet
 * (hipExtLaunchKernel), so tracing adds no packets to the stream.
 * pensieve_trace_read waits for the traced launches still in flight,
 * writes up to max_records records {kernel, work items, milliseconds} in
 * launch order (kernel: 0 kv_append, 1 vector attention, 2 matrix-core
 * attention, 3 split merge, 4 block swap), sets *num_records to the number
 * written, and
 * clears the trace (at most 65536 records are kept between reads).
 * enable > 0 turns tracing on and times every enable-th launch of each kernel
 * kind (1: every launch); 0 turns it off.  A timed launch costs more than an
 * ordinary one (about 15 us of host time with ROCm 7.2, more the first time
 * an event is used), so a loop should warm up traced before it is measured.
 * Enabling fills a pool of reusable events (a few hundred, on the current
 * device).  Tracing is off by default and costs nothing when off.
 */
typedef struct pensieve_trace_record {
  int32_t kernel;
  int32_t items;
  float ms;
} pensieve_trace_record;

pensieve_status pensieve_trace_enable(int32_t enable);
pensieve_status pensieve_trace_read(pensieve_trace_record* records_host, int32_t max_records,
                                    int32_t* num_records);

#ifdef __cplusplus
}
#endif

#endif /* PENSIEVE_H */
