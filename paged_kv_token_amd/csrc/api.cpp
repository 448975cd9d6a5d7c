// C ABI of libpensieve: argument checks, the host work planner, pinned
// staging of the work list, and kernel launches on the caller's stream.
//
// Planning follows the compact work queue of "PersistentKV: Page-Aware
// Decode Scheduling for Long-Context LLM Serving on Commodity GPUs"
// (section 2): the unified batch becomes a dense list of real work items
// (request, KV head, row range, KV partition) with no padding items, ordered
// longest first so the hardware dispatcher balances the tail.  Items with
// many query vectors go to the matrix-core kernel; decode rows and small row
// groups go to the vector kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <unordered_map>
#include <vector>

#include "host_status.h"
#include "launch.h"
#include "pensieve.h"

namespace pk {
LaunchEvents& launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}
}  // namespace pk

namespace {

thread_local std::string g_last_error;

pensieve_status fail(pensieve_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pensieve_status ok() {
  g_last_error.clear();
  return PENSIEVE_OK;
}

pensieve_status hip_fail(hipError_t e, const char* what) {
  return fail(PENSIEVE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kBlockSize = 16;
constexpr int kVectorRowsMax = 8;    // query vectors per vector-kernel item
// Head groups of this size or more always run on the matrix cores.  On decode rows (128 requests
// of 2048 tokens, 8 KV heads, bf16) the matrix-core kernel streams the K/V at 5.8 TB/s for G = 8
// and 5.9 TB/s for G = 4, where the vector kernel, holding G query vectors per lane group,
// reaches 2.7 and 5.5 TB/s.
constexpr int kMatrixMinGroup = 4;
constexpr int kMfmaRows = 128;       // query vectors per matrix-core item (four waves)
// Eight-wave matrix-core items (256 query vectors, one workgroup per CU) replace the four-wave
// ones in calls whose four-wave items would not fill one round of workgroup slots
// (kSplitTargetItems) and hold a request of more than kMfmaRows query vectors per KV head: each
// busy CU then runs two waves per SIMD that share every K/V tile they load, and whole CUs are left
// to the vector items beside them.  Long-context batch (a 512-row prefill beside three decode
// requests): 0.825 -> 0.798 ms.  A call that fills the GPU keeps four-wave items, whose two
// workgroups per CU overlap each other's barriers and load waits (the GQA recompute batch was
// 0.60 -> 0.66 ms with eight-wave items).
constexpr int kWideRows = 256;
constexpr int kWideFlag = 1 << 8;    // Segment / PlannedItem param bit: eight-wave matrix-core items
constexpr int kMaxPartitions = 256;
// Adaptive split-KV of pensieve_attn_fwd: the plan aims at about kSplitTargetItems work
// items of similar length -- one round of the matrix-core kernel, two workgroups on each of
// MI355X's 256 CUs, so that the long requests' items all run at once instead of leaving a
// partial second round; a request whose one item would be longer than that share is cut into
// partitions of at least kSplitMinBlocks blocks (and at least one 64-key tile).
constexpr long long kSplitTargetItems = 512;
constexpr long long kSplitMinBlocks = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int dtype) { return dtype == PENSIEVE_F32 ? 4 : dtype == PENSIEVE_FP8_E4M3 ? 1 : 2; }

// Types of Q / O (and of pools that hold the query type).
bool valid_dtype(int dtype) { return dtype == PENSIEVE_F32 || dtype == PENSIEVE_F16 || dtype == PENSIEVE_BF16; }
// Types a pool may hold.
bool valid_pool_dtype(int dtype) { return valid_dtype(dtype) || dtype == PENSIEVE_FP8_E4M3; }
bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

pensieve_status check_desc(const pensieve_batch_desc* d) {
  if (!d) return fail(PENSIEVE_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_reqs < 0) return fail(PENSIEVE_ERR_INVALID_ARG, "num_reqs < 0");
  if (d->num_heads <= 0 || d->num_kv_heads <= 0)
    return fail(PENSIEVE_ERR_INVALID_ARG, "num_heads and num_kv_heads must be > 0");
  if (d->num_heads % d->num_kv_heads != 0)
    return fail(PENSIEVE_ERR_INVALID_ARG, "num_heads (%d) is not a multiple of num_kv_heads (%d)", d->num_heads,
                d->num_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PENSIEVE_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", d->head_dim);
  if (d->block_size != kBlockSize) return fail(PENSIEVE_ERR_UNSUPPORTED, "block_size %d unsupported (16)", d->block_size);
  if (!valid_dtype(d->dtype)) return fail(PENSIEVE_ERR_UNSUPPORTED, "unknown dtype %d", d->dtype);
  if (d->kv_dtype != d->dtype) {
    if (d->kv_dtype != PENSIEVE_FP8_E4M3)
      return fail(PENSIEVE_ERR_UNSUPPORTED, "kv_dtype %d with dtype %d: pools hold dtype or FP8_E4M3", d->kv_dtype,
                  d->dtype);
    if (d->dtype == PENSIEVE_F32) return fail(PENSIEVE_ERR_UNSUPPORTED, "FP8_E4M3 pools need F16 or BF16 queries");
    if (!valid_scale(d->k_scale) || !valid_scale(d->v_scale))
      return fail(PENSIEVE_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  }
  if (d->num_blocks <= 0) return fail(PENSIEVE_ERR_INVALID_ARG, "num_blocks must be > 0");
  if (d->block_table_stride <= 0) return fail(PENSIEVE_ERR_INVALID_ARG, "block_table_stride must be > 0");
  if (!(d->softmax_scale > 0.f)) return fail(PENSIEVE_ERR_INVALID_ARG, "softmax_scale must be > 0");
  if (d->flags & ~(PENSIEVE_FLAG_VECTOR_ONLY | PENSIEVE_FLAG_NO_SPLIT | PENSIEVE_FLAG_SINGLE_STREAM))
    return fail(PENSIEVE_ERR_INVALID_ARG, "unknown flags 0x%x", d->flags);
  if (d->num_reqs > 0 && (!d->context_lens_host || !d->cu_q_lens_host))
    return fail(PENSIEVE_ERR_INVALID_ARG, "context_lens_host / cu_q_lens_host is NULL");
  if (d->num_reqs > 0 && d->cu_q_lens_host[0] != 0) return fail(PENSIEVE_ERR_INVALID_ARG, "cu_q_lens_host[0] != 0");
  for (int r = 0; r < d->num_reqs; ++r) {
    const int L = d->context_lens_host[r];
    const long q = (long)d->cu_q_lens_host[r + 1] - d->cu_q_lens_host[r];
    if (L < 0) return fail(PENSIEVE_ERR_INVALID_ARG, "context_lens[%d] = %d < 0", r, L);
    if (q < 0) return fail(PENSIEVE_ERR_INVALID_ARG, "cu_q_lens decreases at request %d", r);
    if (q > L) return fail(PENSIEVE_ERR_INVALID_ARG, "request %d has %ld query rows but context length %d", r, q, L);
    const long nblk = ((long)L + kBlockSize - 1) / kBlockSize;
    if (nblk > d->block_table_stride)
      return fail(PENSIEVE_ERR_INVALID_ARG, "request %d needs %ld blocks but block_table_stride is %d", r, nblk,
                  d->block_table_stride);
    if (nblk > (long)d->num_blocks)
      return fail(PENSIEVE_ERR_INVALID_ARG, "request %d needs %ld blocks but the pool has %d", r, nblk, d->num_blocks);
  }
  return PENSIEVE_OK;
}

// ---- planning -------------------------------------------------------------------------
enum Kernel { kVector = 0, kMatrix = 1 };

struct PlannedItem {
  pk::WorkItem w;
  int kernel;
  int param;        // vector: query vectors per item (1,2,4,8); matrix: group size, | kWideFlag
                    // for eight-wave items
  long long cost;
};

struct Segment {
  int kernel;
  int param;
  int begin;
  int count;
};

// Workspace of a plan: [work items | per-request partial base rows | partial row map |
// part_m | part_l | part_o], each 256-byte aligned; the last five exist only when
// pensieve_attn_fwd splits some requests (compact partials: split requests' rows only).
struct Plan {
  std::vector<pk::WorkItem> items;
  std::vector<PlannedItem> planned;   // same order as items
  std::vector<Segment> segments;
  std::vector<int32_t> part_row_base;   // per request: first partial row, -1 if not split
  std::vector<int32_t> rowmap;          // per partial row: {output row, partitions}
  int split_rows = 0, pmax = 1, num_heads = 0, head_dim = 0;
  size_t items_bytes() const { return align_up(items.size() * sizeof(pk::WorkItem)); }
  size_t base_off() const { return items_bytes(); }
  size_t rowmap_off() const { return base_off() + align_up(part_row_base.size() * sizeof(int32_t)); }
  size_t meta_bytes() const { return rowmap_off() + align_up(rowmap.size() * sizeof(int32_t)); }
  size_t partials() const { return (size_t)split_rows * num_heads * pmax; }
  size_t pm_off() const { return meta_bytes(); }
  size_t pl_off() const { return pm_off() + align_up(partials() * sizeof(float)); }
  size_t po_off() const { return pl_off() + align_up(partials() * sizeof(float)); }
  size_t bytes() const {
    return split_rows ? po_off() + align_up(partials() * head_dim * sizeof(float)) : items_bytes();
  }
};

bool matrix_ok(const pensieve_batch_desc* d) {
  const int G = d->num_heads / d->num_kv_heads;
  if (d->dtype == PENSIEVE_F32 || (d->flags & PENSIEVE_FLAG_VECTOR_ONLY)) return false;
  return G >= 1 && G <= 32 && (32 % G) == 0;
}

// Workgroup i of a launch runs on XCD i % kXcds, and each XCD has its own L2.
// Matrix-core items of one (request, KV head, partition) stream the same K/V,
// so they are kept on one XCD: such groups, costliest first, go one by one to
// the least loaded of kXcds bins; each bin then lists its items by cost class,
// longest first, and the bins are interleaved so that bin x occupies launch
// slots x, x + kXcds, ...  Bins are padded to equal length with zero-row
// items, which the kernel leaves at once.
constexpr int kXcds = 8;

// One (request, KV head, partition) of matrix-core items: items[first, first + count).
struct ItemGroup {
  long long cost;   // total over the group's items
  int first, count;
};

// Reorder idx so that key(i) descends, keeping the given order among equal keys: a counting
// sort when the keys span a small range (plan costs in blocks, cost classes), else a
// comparison sort.
template <class Key>
void sort_descending(std::vector<int>& idx, Key key) {
  thread_local std::vector<int> start_tl, tmp_tl;
  std::vector<int>& start = start_tl;
  std::vector<int>& tmp = tmp_tl;
  long long top = 0;
  bool small = true;
  for (int i : idx) {
    const long long k = key(i);
    top = std::max(top, k);
    small = small && k >= 0;
  }
  if (!small || top > 8 * (long long)idx.size() + 4096) {
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return key(a) > key(b); });
    return;
  }
  start.assign((size_t)top + 2, 0);   // bucket b = top - key: the largest key first
  for (int i : idx) start[(size_t)(top - key(i)) + 1]++;
  for (size_t b = 1; b < start.size(); ++b) start[b] += start[b - 1];
  tmp.resize(idx.size());
  for (int i : idx) tmp[start[(size_t)(top - key(i))]++] = i;
  idx.swap(tmp);
}

// Cost class of a work item: three octaves of its length in 64-unit steps,
// floor(log2(cost / 64) / 3).  Narrower classes (one octave) spread a request's items over more
// classes, which run apart in time, so its K/V was fetched again: on the GQA recompute batch the
// matrix-core launch read 717 MB instead of 606 MB and took 1 % longer; wider ones (four and five
// octaves) leave longer items in each bin's last round (3-4 % slower).
int cost_class(long long cost) {
  const unsigned long long steps = (unsigned long long)std::max(1LL, cost / 64);
  return (63 - __builtin_clzll(steps)) / 3;
}

void xcd_order(const std::vector<PlannedItem>& items, const std::vector<ItemGroup>& groups,
               std::vector<PlannedItem>& out) {
  thread_local std::vector<int> order_tl;
  thread_local std::vector<int> bins_tl[kXcds];
  std::vector<int>& order = order_tl;
  order.resize(groups.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  sort_descending(order, [&](int g) { return groups[g].cost / 64; });
  if (items.size() < 2 * kXcds) {
    for (int gi : order)
      out.insert(out.end(), items.begin() + groups[gi].first, items.begin() + groups[gi].first + groups[gi].count);
    return;
  }
  std::vector<int>* const bins = bins_tl;
  for (int x = 0; x < kXcds; ++x) bins[x].clear();
  long long load[kXcds] = {};
  for (int gi : order) {
    int x = 0;
    for (int y = 1; y < kXcds; ++y)
      if (load[y] < load[x]) x = y;
    load[x] += groups[gi].cost;
    for (int k = 0; k < groups[gi].count; ++k) bins[x].push_back(groups[gi].first + k);
  }
  // Each XCD runs its items by cost class, longest class first (items of a request differ when
  // its rows sit at very different positions, e.g. recomputed leading rows), so that its last
  // round holds its shortest items.  Inside a class the items keep the order above, a request's
  // items next to each other, so that they run close together in time and share its K/V in the
  // XCD's L2.
  for (int x = 0; x < kXcds; ++x)
    sort_descending(bins[x], [&](int i) { return (long long)cost_class(items[i].cost); });
  size_t longest = 0;
  for (int x = 0; x < kXcds; ++x) longest = std::max(longest, bins[x].size());
  PlannedItem filler = items.front();
  filler.w.q_count = 0;
  filler.cost = 0;
  out.reserve(out.size() + longest * kXcds);
  for (size_t k = 0; k < longest; ++k)
    for (int x = 0; x < kXcds; ++x) out.push_back(k < bins[x].size() ? items[bins[x][k]] : filler);
}

// Kernel of a request's items: the vector kernel for few query vectors of small head groups.
bool routes_to_matrix(bool matrix_allowed, int q, int G) {
  return matrix_allowed && ((long long)q * G > kVectorRowsMax || G >= kMatrixMinGroup);
}

// Work items of one request for one KV head and partition (no split): matrix-core items of
// kMfmaRows query vectors, or vector items of at most kVectorRowsMax.
long long items_per_kv_head(int q, int G, bool use_matrix) {
  if (use_matrix) return (q + kMfmaRows / G - 1) / (kMfmaRows / G);
  const int heads_per = std::min(G, kVectorRowsMax);
  const int tok_per = std::max(1, kVectorRowsMax / heads_per);
  return (long long)((G + heads_per - 1) / heads_per) * ((q + tok_per - 1) / tok_per);
}

// Partitions per request.  num_partitions >= 1: that many for every request (the explicit
// split-KV pair).  0 (pensieve_attn_fwd): adaptive; an item's length is taken as its
// request's block count, the fair share is the total over all items divided by
// kSplitTargetItems, and a request is cut only when its items are longer than the share.
std::vector<int> choose_partitions(const pensieve_batch_desc* d, int num_partitions) {
  std::vector<int> P(d->num_reqs, num_partitions >= 1 ? num_partitions : 1);
  if (num_partitions >= 1 || (d->flags & PENSIEVE_FLAG_NO_SPLIT)) return P;
  const int G = d->num_heads / d->num_kv_heads;
  const bool mat = matrix_ok(d);
  long long total = 0;
  for (int r = 0; r < d->num_reqs; ++r) {
    const int q = d->cu_q_lens_host[r + 1] - d->cu_q_lens_host[r];
    if (q == 0) continue;
    const long long nblk = (d->context_lens_host[r] + kBlockSize - 1) / kBlockSize;
    const bool use_matrix = routes_to_matrix(mat, q, G);
    total += items_per_kv_head(q, G, use_matrix) * d->num_kv_heads * (nblk + 1);
  }
  const long long share = std::max(kSplitMinBlocks, total / kSplitTargetItems);
  // When the matrix-core items leave CUs free, the vector items run beside them on a second
  // stream, in whatever workgroup slots are left: vector requests then get twice the items.
  long long matrix_items = 0;
  bool any_vector = false;
  for (int r = 0; r < d->num_reqs; ++r) {
    const int q = d->cu_q_lens_host[r + 1] - d->cu_q_lens_host[r];
    if (q == 0) continue;
    if (routes_to_matrix(mat, q, G)) matrix_items += items_per_kv_head(q, G, true) * d->num_kv_heads;
    else any_vector = true;
  }
  const bool beside = any_vector && matrix_items > 0 && matrix_items < kSplitTargetItems;
  const long long vshare = beside ? std::max(kSplitMinBlocks, total / (2 * kSplitTargetItems)) : share;
  for (int r = 0; r < d->num_reqs; ++r) {
    const int q = d->cu_q_lens_host[r + 1] - d->cu_q_lens_host[r];
    const long long nblk = (d->context_lens_host[r] + kBlockSize - 1) / kBlockSize;
    const long long sh = (q > 0 && routes_to_matrix(mat, q, G)) ? share : vshare;
    if (q == 0 || nblk + 1 <= sh) continue;
    const long long want = (nblk + 1 + sh - 1) / sh;
    P[r] = (int)std::max(1LL, std::min({want, (long long)kMaxPartitions, nblk / 4}));
  }
  return P;
}

void build_plan(const pensieve_batch_desc* d, int num_partitions, Plan& plan) {
  const int G = d->num_heads / d->num_kv_heads;
  const bool mat = matrix_ok(d);
  const std::vector<int> parts = choose_partitions(d, num_partitions);
  plan.part_row_base.clear();
  plan.rowmap.clear();
  plan.split_rows = 0;
  plan.pmax = 1;
  plan.num_heads = d->num_heads;
  plan.head_dim = d->head_dim;
  if (num_partitions == 0) {
    for (int r = 0; r < d->num_reqs; ++r) {
      if (parts[r] <= 1) continue;
      if (plan.part_row_base.empty()) plan.part_row_base.assign(d->num_reqs, -1);
      plan.part_row_base[r] = plan.split_rows;
      for (int i = d->cu_q_lens_host[r]; i < d->cu_q_lens_host[r + 1]; ++i) {
        plan.rowmap.push_back(i);
        plan.rowmap.push_back(parts[r]);
      }
      plan.split_rows += d->cu_q_lens_host[r + 1] - d->cu_q_lens_host[r];
      plan.pmax = std::max(plan.pmax, parts[r]);
    }
  }
  // Requests longest first (by KV blocks), so that every list below comes out longest first
  // without sorting its items.
  // Scratch lists keep their capacity from call to call (one set per host thread).
  thread_local std::vector<int> reqs;
  thread_local std::vector<PlannedItem> mat_items;
  thread_local std::vector<ItemGroup> groups;
  thread_local std::vector<PlannedItem> vec[4];   // vector items by width 1, 2, 4, 8 query vectors
  reqs.clear();
  mat_items.clear();
  groups.clear();
  for (auto& v : vec) v.clear();
  for (int r = 0; r < d->num_reqs; ++r)
    if (d->cu_q_lens_host[r + 1] > d->cu_q_lens_host[r]) reqs.push_back(r);
  std::stable_sort(reqs.begin(), reqs.end(),
                   [&](int a, int b) { return d->context_lens_host[a] > d->context_lens_host[b]; });
  bool wide = false;
  if (mat && (d->kv_dtype != PENSIEVE_FP8_E4M3 || d->head_dim == 128)) {   // kernels that exist
    long long narrow_items = 0;
    bool long_rows = false;
    for (int r : reqs) {
      const int q = d->cu_q_lens_host[r + 1] - d->cu_q_lens_host[r];
      if (!routes_to_matrix(mat, q, G)) continue;
      narrow_items += items_per_kv_head(q, G, true) * d->num_kv_heads * parts[r];
      long_rows = long_rows || (long long)q * G > kMfmaRows;
    }
    wide = long_rows && narrow_items < kSplitTargetItems;
  }
  const int mat_rows = wide ? kWideRows : kMfmaRows;
  for (int r : reqs) {
    const int L = d->context_lens_host[r];
    const int q = d->cu_q_lens_host[r + 1] - d->cu_q_lens_host[r];
    const int P = parts[r];
    const long long nblk = (L + kBlockSize - 1) / kBlockSize;
    const long long per = (nblk + P - 1) / P;
    const bool use_matrix = routes_to_matrix(mat, q, G);
    for (int part = 0; part < P; ++part) {
      const long long blocks = std::max(0LL, std::min(per, nblk - part * per));
      for (int g = 0; g < d->num_kv_heads; ++g) {
        if (use_matrix) {
          const int tok_tile = mat_rows / G;
          groups.push_back({0, (int)mat_items.size(), 0});
          for (int q0 = 0; q0 < q; q0 += tok_tile) {
            PlannedItem p{};
            const int qc = std::min(tok_tile, q - q0);
            p.w = {r, q0, qc, g, 0, G, part, P};
            p.kernel = kMatrix;
            p.param = G | (wide ? kWideFlag : 0);
            // An item streams the keys of its partition that its last (largest) position can
            // see, plus a fixed cost of about one block.
            const long long last = d->q_pos_host ? (long long)d->q_pos_host[d->cu_q_lens_host[r] + q0 + qc - 1]
                                                 : (long long)L - q + q0 + qc - 1;
            const long long seen = std::min(std::max(std::min(last + 1, (long long)L) - part * per * kBlockSize, 0LL),
                                            blocks * kBlockSize);
            p.cost = ((seen + kBlockSize - 1) / kBlockSize + 1) * 64;
            mat_items.push_back(p);
            groups.back().cost += p.cost;
            groups.back().count++;
          }
        } else {
          const int heads_per = std::min(G, kVectorRowsMax);
          const int tok_per = std::max(1, kVectorRowsMax / heads_per);
          for (int h0 = 0; h0 < G; h0 += heads_per) {
            const int hc = std::min(heads_per, G - h0);
            for (int q0 = 0; q0 < q; q0 += tok_per) {
              const int qc = std::min(tok_per, q - q0);
              PlannedItem p{};
              p.w = {r, q0, qc, g, h0, hc, part, P};
              p.kernel = kVector;
              p.param = next_pow2(qc * hc);
              p.cost = (blocks + 1) * (4 + qc * hc);
              vec[p.param == 1 ? 0 : p.param == 2 ? 1 : p.param == 4 ? 2 : 3].push_back(p);
            }
          }
        }
      }
    }
  }
  // Launch order: the matrix-core segment (spread over the XCDs), then vector items by width.
  std::vector<PlannedItem>& ordered = plan.planned;
  ordered.clear();
  if (!mat_items.empty()) xcd_order(mat_items, groups, ordered);
  for (auto& v : vec) ordered.insert(ordered.end(), v.begin(), v.end());
  plan.items.clear();
  plan.items.reserve(ordered.size());
  plan.segments.clear();
  for (size_t i = 0; i < ordered.size(); ++i) {
    plan.items.push_back(ordered[i].w);
    if (plan.segments.empty() || plan.segments.back().kernel != ordered[i].kernel ||
        plan.segments.back().param != ordered[i].param) {
      plan.segments.push_back({ordered[i].kernel, ordered[i].param, (int)i, 0});
    }
    plan.segments.back().count++;
  }
}

// ---- pinned staging of work lists ---------------------------------------------------------
// Each device gets a small ring of page-locked, device-mapped host buffers; a
// work list is copied into the next one and pulled into the workspace by a
// small copy kernel on the caller's stream (one queue, no copy-engine handoff).
// A buffer is refilled only after the work that read it has finished: the copy
// kernel's per-workgroup flags say so for work lists, an event for swap block
// lists (read by the swap kernel itself).
struct Stager {
  static constexpr int kSlots = 32;   // deep enough that a long swap does not hold up later calls
  // Every slot starts as a slice of one page-locked slab, so that the first pass over the ring
  // allocates nothing (a page-locked free synchronises the device); only a work list longer
  // than a slice gives its slot a buffer of its own.
  static constexpr size_t kSlotBytes = 512 * 1024;
  struct Slot {
    void* host = nullptr;
    void* mapped = nullptr;   // the same buffer as seen from the device
    size_t cap = 0;
    bool owned = false;       // a buffer of its own (else a slice of the slab)
    hipEvent_t ev = nullptr;
    bool pending = false;
    bool in_use = false;      // handed out by stage_acquire, not yet given back by stage_release
    // The slot's last use is over once every one of the flag_blocks workgroups of the copy
    // kernel that read it has stored `seq` into its flag; with no such kernel (flag_blocks == 0)
    // once `ev` has completed.
    uint32_t seq = 0;
    int flag_blocks = 0;
    uint32_t* flags_host = nullptr;   // kStageCopyBlocks words of the flag array
    uint32_t* flags_dev = nullptr;    // the same words as seen from the device
  };
  std::mutex mu;
  Slot slots[kSlots];
  int next = 0;
  void* slab = nullptr;
  uint32_t* flags = nullptr;          // kSlots x kStageCopyBlocks words, page-locked and coherent
  uint32_t seq = 0;                   // last sequence number handed out (0 is never used)
};

std::mutex g_stagers_mu;
std::unordered_map<int, Stager*> g_stagers;

Stager* stager_for_current_device(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_stagers_mu);
  auto it = g_stagers.find(dev);
  if (it != g_stagers.end()) return it->second;
  Stager* s = new Stager();
  g_stagers[dev] = s;
  return s;
}

// Wait until every workgroup of the copy kernel that last read slot `s` has stored the slot's
// sequence number (no event on the stream: an event recorded between two kernels holds the next
// one back by about 5 us).  Bounded: if the flags have not all arrived within two seconds
// (PENSIEVE_STAGE_WAIT_US microseconds when set, read at each wait), the device is synchronised
// once, after which every launch enqueued before has finished; flags still missing then are an
// error, not a hang.
hipError_t wait_stage_flags(const Stager::Slot& s) {
  auto arrived = [&s] {
    for (int b = 0; b < s.flag_blocks; ++b)
      if (__atomic_load_n(s.flags_host + b, __ATOMIC_ACQUIRE) != s.seq) return false;
    return true;
  };
  if (arrived()) return hipSuccess;
  long long limit_us = 2000000;
  if (const char* v = std::getenv("PENSIEVE_STAGE_WAIT_US"); v && *v) limit_us = std::max(0LL, std::atoll(v));
  const auto t0 = std::chrono::steady_clock::now();
  for (unsigned spin = 0; !arrived(); ++spin) {
    if (spin % 1024 == 0) {
      if (std::chrono::steady_clock::now() - t0 >= std::chrono::microseconds(limit_us)) {
        const hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return e;
        return arrived() ? hipSuccess : hipErrorUnknown;
      }
      std::this_thread::yield();
    }
  }
  return hipSuccess;
}

// Copy `bytes` from `src` into the next staging buffer of this device (waiting until the
// buffer's previous use on the GPU has finished) and return its device mapping; the caller
// enqueues the work that reads it, then calls stage_release on the same stream.
hipError_t stage_acquire(const void* src, size_t bytes, void** mapped, Stager::Slot** slot_out) {
  hipError_t e;
  Stager* st = stager_for_current_device(&e);
  if (!st) return e;
  std::unique_lock<std::mutex> lk(st->mu);
  if (!st->slab) {
    void* slab = nullptr;
    void* slab_mapped = nullptr;
    void* flags = nullptr;
    void* flags_mapped = nullptr;
    constexpr size_t kFlagBytes = Stager::kSlots * pk::kStageCopyBlocks * sizeof(uint32_t);
    if ((e = hipHostMalloc(&slab, Stager::kSlots * Stager::kSlotBytes, hipHostMallocMapped)) != hipSuccess)
      return e;
    if ((e = hipHostGetDevicePointer(&slab_mapped, slab, 0)) != hipSuccess ||
        (e = hipHostMalloc(&flags, kFlagBytes, hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess ||
        (e = hipHostGetDevicePointer(&flags_mapped, flags, 0)) != hipSuccess) {
      if (flags) (void)hipHostFree(flags);
      (void)hipHostFree(slab);
      return e;
    }
    std::memset(flags, 0, kFlagBytes);
    st->slab = slab;
    st->flags = static_cast<uint32_t*>(flags);
    for (int i = 0; i < Stager::kSlots; ++i) {
      st->slots[i].host = static_cast<uint8_t*>(st->slab) + i * Stager::kSlotBytes;
      st->slots[i].mapped = static_cast<uint8_t*>(slab_mapped) + i * Stager::kSlotBytes;
      st->slots[i].cap = Stager::kSlotBytes;
      st->slots[i].flags_host = st->flags + i * pk::kStageCopyBlocks;
      st->slots[i].flags_dev = static_cast<uint32_t*>(flags_mapped) + i * pk::kStageCopyBlocks;
    }
  }
  // The next slot that no other call holds between its acquire and its release.  When calls on
  // other threads hold every slot, this one retries (without the lock) for up to ten seconds.
  int pick = -1;
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    for (int k = 0; k < Stager::kSlots && pick < 0; ++k) {
      const int i = (st->next + k) % Stager::kSlots;
      if (!st->slots[i].in_use) pick = i;
    }
    if (pick >= 0) break;
    if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(10)) return hipErrorNotReady;
    lk.unlock();
    std::this_thread::yield();
    lk.lock();
  }
  Stager::Slot& s = st->slots[pick];
  st->next = (pick + 1) % Stager::kSlots;
  s.in_use = true;   // reserved: no other call takes it while this one waits; every failure below frees it
  auto give_back = [&s](hipError_t err) {
    s.in_use = false;
    return err;
  };
  if (s.pending) {
    // The wait runs without the lock, so that calls on other threads can take other slots meanwhile.
    lk.unlock();
    e = s.flag_blocks > 0 ? wait_stage_flags(s) : hipEventSynchronize(s.ev);
    lk.lock();
    if (e != hipSuccess) return give_back(e);
    s.pending = false;
  }
  if (s.cap < bytes) {
    if (s.owned && (e = hipHostFree(s.host)) != hipSuccess) return give_back(e);
    s.host = nullptr;
    s.mapped = nullptr;
    s.cap = 0;            // stays empty if the allocation below fails
    s.owned = false;
    size_t cap = 2 * Stager::kSlotBytes;
    while (cap < bytes) cap *= 2;
    if ((e = hipHostMalloc(&s.host, cap, hipHostMallocMapped)) != hipSuccess) {
      s.host = nullptr;
      return give_back(e);
    }
    if ((e = hipHostGetDevicePointer(&s.mapped, s.host, 0)) != hipSuccess) {
      (void)hipHostFree(s.host);
      s.host = nullptr;
      s.mapped = nullptr;
      return give_back(e);
    }
    s.cap = cap;
    s.owned = true;
  }
  if (!s.ev && (e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming)) != hipSuccess) return give_back(e);
  std::memcpy(s.host, src, bytes);
  if (++st->seq == 0) st->seq = 1;
  s.seq = st->seq;
  s.flag_blocks = 0;
  *mapped = s.mapped;
  *slot_out = &s;
  return hipSuccess;
}

// The staging buffer may be reused once `stream` has passed this point, or, when `flag_blocks`
// workgroups of a copy kernel read it and store the slot's sequence number when done, once they
// all have.  If the event cannot be recorded the slot stays held: nothing would tell when the
// work that reads the buffer is done.
hipError_t stage_release(Stager::Slot* slot, hipStream_t stream, int flag_blocks = 0) {
  hipError_t e;
  Stager* st = stager_for_current_device(&e);
  if (!st) return e;
  std::lock_guard<std::mutex> lk(st->mu);
  if (flag_blocks == 0 && (e = hipEventRecord(slot->ev, stream)) != hipSuccess) return e;
  slot->flag_blocks = flag_blocks;
  slot->in_use = false;
  slot->pending = true;
  return hipSuccess;
}

// How a plan's work list reaches the device.
enum class Upload {
  kStaged,     // the pinned staging ring (allocated by the library on first use) and a copy kernel
  kPageable,   // a plain host-to-device copy from pageable host memory; allocates nothing
};

// Host-visible misuse: the staged work lists and the library's side stream do not survive
// graph capture (a captured graph would replay a stale list), so capture is refused.
pensieve_status refuse_capture(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e, "stream capture query");
  if (cs != hipStreamCaptureStatusNone)
    return fail(PENSIEVE_ERR_UNSUPPORTED, "the stream is being captured into a graph; the calls plan and upload "
                                          "their work list at every call and cannot be captured");
  return PENSIEVE_OK;
}

// ---- per-launch timing trace ------------------------------------------------------------
// While tracing is on, every launch records start/stop events through its own dispatch packet.
// Launches still in flight keep their events in g_pending; finished ones are turned into
// records (and their events recycled) whenever a new launch is traced, so only a few dozen
// events are ever live and none are created inside a timed loop once the pool is warm.

enum TraceKernel { kTraceAppend = 0, kTraceVector = 1, kTraceMatrix = 2, kTraceMerge = 3, kTraceSwap = 4 };

struct TraceEntry {
  int kernel;
  int items;
  hipEvent_t start, stop;
};

std::mutex g_trace_mu;
bool g_trace_on = false;
int g_trace_every = 1;                // time every n-th launch of each kernel kind
long long g_trace_seen[5] = {};  // launches per kernel kind (TraceKernel) since tracing was enabled
std::deque<TraceEntry> g_pending;
std::vector<pensieve_trace_record> g_records;
hipError_t g_trace_error = hipSuccess;
std::vector<hipEvent_t> g_event_pool;
constexpr size_t kMaxTraceEntries = 1 << 16;
constexpr size_t kTracePoolWarm = 256;

hipEvent_t trace_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Turn one traced launch into a record and recycle its events (g_trace_mu held).
void finish_entry(const TraceEntry& t) {
  float ms = 0.f;
  const hipError_t e = hipEventElapsedTime(&ms, t.start, t.stop);
  if (e != hipSuccess && g_trace_error == hipSuccess) g_trace_error = e;
  if (g_records.size() < kMaxTraceEntries) g_records.push_back({t.kernel, t.items, ms});
  g_event_pool.push_back(t.start);
  g_event_pool.push_back(t.stop);
}

// Collect the launches that have finished, oldest first (g_trace_mu held).
void harvest_finished() {
  while (!g_pending.empty() && hipEventQuery(g_pending.front().stop) == hipSuccess) {
    finish_entry(g_pending.front());
    g_pending.pop_front();
  }
}

// Times the one launch made while it is alive: the launch itself records the events (its
// dispatch packet carries them, hipExtLaunchKernel), so timing adds no packets to the stream.
struct TraceScope {
  bool active = false;
  TraceEntry entry{};
  TraceScope(int kernel, int items, hipStream_t) {
    std::lock_guard<std::mutex> lk(g_trace_mu);
    if (!g_trace_on) return;
    if (g_trace_seen[kernel]++ % g_trace_every != 0) return;
    harvest_finished();
    if (g_records.size() + g_pending.size() >= kMaxTraceEntries) return;
    entry = {kernel, items, trace_event(), trace_event()};
    if (!entry.start || !entry.stop) {   // keep whichever event was made for a later launch
      if (entry.start) g_event_pool.push_back(entry.start);
      if (entry.stop) g_event_pool.push_back(entry.stop);
      return;
    }
    pk::launch_events() = {entry.start, entry.stop};
    active = true;
  }
  ~TraceScope() {
    if (!active) return;
    pk::launch_events() = {};
    std::lock_guard<std::mutex> lk(g_trace_mu);
    g_pending.push_back(entry);
  }
};

// Side stream and fork/join events per device: when a plan has both
// matrix-core and vector items, the vector segments run on the side stream
// concurrently with the matrix-core segment (they touch disjoint requests and
// outputs), and the caller's stream waits for both.
struct Concurrency {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_conc_mu;
std::unordered_map<int, Concurrency> g_conc;

hipError_t concurrency_for_current_device(Concurrency** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_conc_mu);
  Concurrency& c = g_conc[dev];
  if (!c.side) {   // all three or none: a partial set is destroyed and the next call tries again
    Concurrency n;
    if ((e = hipStreamCreateWithFlags(&n.side, hipStreamNonBlocking)) == hipSuccess &&
        (e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming)) == hipSuccess &&
        (e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming)) == hipSuccess) {
      c = n;
    } else {
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.side) (void)hipStreamDestroy(n.side);
      return e;
    }
  }
  *out = &c;
  return hipSuccess;
}

int device_cu_count() {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev] = n;
  return n;
}

// A work list in a staging buffer, given back after the call's last launch on every return path.
// Its reuse waits for the copy kernel's flags when the copy was launched (`flag_blocks`
// workgroups), else for an event recorded on the caller's stream at the release.
struct StagedList {
  Stager::Slot* slot = nullptr;
  hipStream_t stream = nullptr;
  int flag_blocks = 0;
  hipError_t release() {
    if (!slot) return hipSuccess;
    Stager::Slot* s = slot;
    slot = nullptr;
    return stage_release(s, stream, flag_blocks);
  }
  ~StagedList() { (void)release(); }
};

pensieve_status run_plan(const pensieve_batch_desc* d, const Plan& plan, pk::AttnArgs& args, void* workspace,
                         hipStream_t stream, Upload upload = Upload::kStaged) {
  uint8_t* const ws = static_cast<uint8_t*>(workspace);
  StagedList staged;
  staged.stream = stream;
  const uint8_t* const meta_dev = ws;   // the work list as the kernels read it
  auto to_device = [&](const void* src, size_t bytes) -> hipError_t {
    if (bytes == 0) return hipSuccess;
    if (upload == Upload::kPageable)   // pageable source: the copy has taken the bytes when the call returns
      return hipMemcpyAsync(ws, src, bytes, hipMemcpyHostToDevice, stream);
    void* mapped = nullptr;
    hipError_t e = stage_acquire(src, bytes, &mapped, &staged.slot);
    if (e != hipSuccess) return e;
    if (bytes % 16 == 0)
      return pk::launch_stage_copy(mapped, ws, bytes, stream, staged.slot->flags_dev, staged.slot->seq,
                                   &staged.flag_blocks);
    return hipMemcpyAsync(ws, staged.slot->host, bytes, hipMemcpyHostToDevice, stream);
  };
  hipError_t e;
  if (plan.split_rows == 0) {
    e = to_device(plan.items.data(), plan.items.size() * sizeof(pk::WorkItem));
  } else {
    // Items, partial base rows and the partial row map go up in one copy; the partials of
    // the split requests live in the rest of the workspace and are merged at the end.
    std::vector<uint8_t> meta(plan.meta_bytes(), 0);
    std::memcpy(meta.data(), plan.items.data(), plan.items.size() * sizeof(pk::WorkItem));
    std::memcpy(meta.data() + plan.base_off(), plan.part_row_base.data(), plan.part_row_base.size() * sizeof(int32_t));
    std::memcpy(meta.data() + plan.rowmap_off(), plan.rowmap.data(), plan.rowmap.size() * sizeof(int32_t));
    e = to_device(meta.data(), meta.size());
    args.part_row_base = reinterpret_cast<const int32_t*>(meta_dev + plan.base_off());
    args.part_m = reinterpret_cast<float*>(ws + plan.pm_off());
    args.part_l = reinterpret_cast<float*>(ws + plan.pl_off());
    args.part_o = reinterpret_cast<float*>(ws + plan.po_off());
    args.part_stride = plan.pmax;
  }
  if (e != hipSuccess) return hip_fail(e, "work-list upload");
  const pk::WorkItem* dev_items = reinterpret_cast<const pk::WorkItem*>(meta_dev);
  bool has_matrix = false, has_vector = false;
  for (const Segment& s : plan.segments) (s.kernel == kMatrix ? has_matrix : has_vector) = true;
  Concurrency* conc = nullptr;
  // Overlap only when the matrix-core items alone cannot occupy every CU (two four-wave
  // workgroups or one eight-wave workgroup per CU); otherwise the kernels just contend for CUs.
  int matrix_items = 0;
  for (const Segment& s : plan.segments)
    if (s.kernel == kMatrix) matrix_items += s.count * ((s.param & kWideFlag) ? 2 : 1);
  // Single-stream mode (the flag, or a call that must allocate nothing, since the side stream is
  // created on first use) keeps every launch on the caller's stream.
  const bool single = (d->flags & PENSIEVE_FLAG_SINGLE_STREAM) || upload == Upload::kPageable;
  const bool fork = !single && has_matrix && has_vector && matrix_items < 2 * device_cu_count();
  std::unique_lock<std::mutex> side_lock;
  if (fork) {
    if ((e = concurrency_for_current_device(&conc)) != hipSuccess) return hip_fail(e, "side stream");
    side_lock = std::unique_lock<std::mutex>(g_conc_mu);   // one fork/join at a time per process
    if ((e = hipEventRecord(conc->fork, stream)) != hipSuccess) return hip_fail(e, "fork event");
    if ((e = hipStreamWaitEvent(conc->side, conc->fork, 0)) != hipSuccess) return hip_fail(e, "fork wait");
  }
  for (const Segment& s : plan.segments) {
    pk::AttnArgs a = args;
    a.items = dev_items + s.begin;
    a.num_items = s.count;
    const hipStream_t st = (fork && s.kernel == kVector) ? conc->side : stream;
    TraceScope trace(s.kernel == kMatrix ? kTraceMatrix : kTraceVector, s.count, st);
    if (s.kernel == kMatrix)
      e = pk::launch_attn_mfma(a, d->dtype, d->kv_dtype, d->head_dim, s.param & (kWideFlag - 1),
                               (s.param & kWideFlag) != 0, st);
    else
      e = pk::launch_attn_vector(a, d->dtype, d->kv_dtype, d->head_dim, s.param, st);
    if (e != hipSuccess) return hip_fail(e, s.kernel == kMatrix ? "matrix-core attention launch" : "vector attention launch");
  }
  if (fork) {
    if ((e = hipEventRecord(conc->join, conc->side)) != hipSuccess) return hip_fail(e, "join event");
    if ((e = hipStreamWaitEvent(stream, conc->join, 0)) != hipSuccess) return hip_fail(e, "join wait");
  }
  if (plan.split_rows > 0) {
    const int rows = plan.split_rows * d->num_heads;
    TraceScope trace(kTraceMerge, rows, stream);
    e = pk::launch_split_merge(args.part_o, args.part_m, args.part_l, rows, d->num_heads, d->head_dim, plan.pmax,
                               reinterpret_cast<const int32_t*>(meta_dev + plan.rowmap_off()), d->dtype, args.o, stream);
    if (e != hipSuccess) return hip_fail(e, "split merge launch");
  }
  if ((e = staged.release()) != hipSuccess) return hip_fail(e, "staging buffer release");
  return ok();
}

pk::AttnArgs make_args(const pensieve_batch_desc* d, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* bt, const int32_t* ctx, const int32_t* cu, const int32_t* q_pos) {
  pk::AttnArgs a{};
  a.q = static_cast<const uint8_t*>(q);
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.block_tables = bt;
  a.context_lens = ctx;
  a.cu_q_lens = cu;
  a.q_pos = q_pos;
  a.num_heads = d->num_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.bt_stride = d->block_table_stride;
  // E4M3 pools: the kernels take q.k over the stored codes, so the K scale joins the softmax
  // scale, and the V scale multiplies the normalised output.
  const bool f8 = d->kv_dtype == PENSIEVE_FP8_E4M3;
  a.scale = d->softmax_scale * (f8 ? d->k_scale : 1.f);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.v_scale = f8 ? d->v_scale : 1.f;
  return a;
}

int total_q(const pensieve_batch_desc* d) { return d->num_reqs > 0 ? d->cu_q_lens_host[d->num_reqs] : 0; }

pensieve_status check_attn_pointers(const pensieve_batch_desc* d, const void* q, const void* k_pool,
                                    const void* v_pool, const int32_t* bt, const int32_t* ctx, const int32_t* cu) {
  if (total_q(d) == 0) return PENSIEVE_OK;
  if (!q || !k_pool || !v_pool || !bt || !ctx || !cu)
    return fail(PENSIEVE_ERR_INVALID_ARG, "a device pointer (q, pools, block_tables, context_lens, cu_q_lens) is NULL");
  return PENSIEVE_OK;
}

// Device address of page-locked host memory (hipHostMalloc / pinned allocations), or null.
void* mapped_host_pointer(void* host) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost) return nullptr;
  return attr.devicePointer;
}

pensieve_status kv_swap(bool to_host, void* k_pool, void* v_pool, int32_t num_blocks, void* k_host, void* v_host,
                        int32_t num_host_blocks, const int32_t* src_blocks_host, const int32_t* dst_blocks_host,
                        int32_t n, int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void* stream) {
  if (n < 0) return fail(PENSIEVE_ERR_INVALID_ARG, "n < 0");
  if (num_kv_heads <= 0) return fail(PENSIEVE_ERR_INVALID_ARG, "num_kv_heads must be > 0");
  if (head_dim != 64 && head_dim != 128) return fail(PENSIEVE_ERR_UNSUPPORTED, "head_dim %d unsupported", head_dim);
  if (!valid_pool_dtype(dtype)) return fail(PENSIEVE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (num_blocks <= 0 || num_host_blocks <= 0) return fail(PENSIEVE_ERR_INVALID_ARG, "pool sizes must be > 0");
  if (n == 0) return ok();
  if (!k_pool || !v_pool || !k_host || !v_host) return fail(PENSIEVE_ERR_INVALID_ARG, "a pool pointer is NULL");
  if (!src_blocks_host || !dst_blocks_host) return fail(PENSIEVE_ERR_INVALID_ARG, "a block list is NULL");
  const int32_t n_src = to_host ? num_blocks : num_host_blocks;
  const int32_t n_dst = to_host ? num_host_blocks : num_blocks;
  std::vector<int32_t> pairs(2 * (size_t)n);
  std::vector<uint8_t> taken(n_dst, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t sb = src_blocks_host[i], db = dst_blocks_host[i];
    if (sb < 0 || sb >= n_src) return fail(PENSIEVE_ERR_INVALID_ARG, "source block %d at %d out of range", sb, i);
    if (db < 0 || db >= n_dst) return fail(PENSIEVE_ERR_INVALID_ARG, "destination block %d at %d out of range", db, i);
    if (taken[db]) return fail(PENSIEVE_ERR_INVALID_ARG, "destination block %d appears twice", db);
    taken[db] = 1;
    pairs[2 * i] = sb;
    pairs[2 * i + 1] = db;
  }
  void* k_map = mapped_host_pointer(k_host);
  void* v_map = mapped_host_pointer(v_host);
  if (!k_map || !v_map)
    return fail(PENSIEVE_ERR_INVALID_ARG, "k_host / v_host must be page-locked host memory mapped for the device");
  const int64_t block_bytes = (int64_t)num_kv_heads * kBlockSize * head_dim * elem_bytes(dtype);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (pensieve_status s = refuse_capture(st); s != PENSIEVE_OK) return s;
  void* pairs_map = nullptr;
  Stager::Slot* slot = nullptr;
  hipError_t e = stage_acquire(pairs.data(), pairs.size() * sizeof(int32_t), &pairs_map, &slot);
  if (e != hipSuccess) return hip_fail(e, "block list staging");
  {
    TraceScope trace(kTraceSwap, n, st);
    e = to_host ? pk::launch_kv_swap(k_pool, v_pool, k_map, v_map, static_cast<const int32_t*>(pairs_map), n,
                                     block_bytes, st)
                : pk::launch_kv_swap(k_map, v_map, k_pool, v_pool, static_cast<const int32_t*>(pairs_map), n,
                                     block_bytes, st);
  }
  const hipError_t e2 = stage_release(slot, st);   // gives the slot back even after a failed launch
  if (e != hipSuccess) return hip_fail(e, "kv swap launch");
  if (e2 != hipSuccess) return hip_fail(e2, "block list staging");
  return ok();
}

// ---- device-contract validator (PENSIEVE_DEBUG=1) -------------------------------------------
// The contents of device arrays are the caller's contract: slots and block ids in range, no
// duplicate slot in one append, host copies equal to the device arrays, query positions strictly
// increasing within a request and below its context length.  With PENSIEVE_DEBUG=1 in the
// environment every append and attention call first copies those arrays to the host (waiting for
// the stream) and returns INVALID_ARG on a violation, before anything of the call is enqueued.
// It reads metadata only, never the pools; it is for tests and debugging, not the hot path.
bool debug_validation() {
  const char* v = std::getenv("PENSIEVE_DEBUG");
  return v && v[0] == '1' && v[1] == '\0';
}

hipError_t fetch_i32(std::vector<int32_t>& out, const int32_t* dev, size_t n, hipStream_t stream) {
  out.assign(n, 0);
  if (n == 0) return hipSuccess;
  hipError_t e = hipMemcpyAsync(out.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(stream);
}

pensieve_status validate_slots(const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                               hipStream_t stream) {
  std::vector<int32_t> slots;
  hipError_t e = fetch_i32(slots, slot_mapping, (size_t)num_tokens, stream);
  if (e != hipSuccess) return hip_fail(e, "debug validation: reading slot_mapping");
  const long long limit = (long long)num_blocks * kBlockSize;
  std::vector<int32_t> used;
  for (int32_t t = 0; t < num_tokens; ++t) {
    if (slots[t] < 0) continue;
    if (slots[t] >= limit)
      return fail(PENSIEVE_ERR_INVALID_ARG, "PENSIEVE_DEBUG: slot_mapping[%d] = %d is past the pool (%lld slots)", t,
                  slots[t], limit);
    used.push_back(slots[t]);
  }
  std::sort(used.begin(), used.end());
  for (size_t i = 1; i < used.size(); ++i)
    if (used[i] == used[i - 1])
      return fail(PENSIEVE_ERR_INVALID_ARG, "PENSIEVE_DEBUG: slot %d appears twice in slot_mapping", used[i]);
  return PENSIEVE_OK;
}

pensieve_status validate_batch(const pensieve_batch_desc* d, const int32_t* block_tables, const int32_t* context_lens,
                               const int32_t* cu_q_lens, const int32_t* q_pos, hipStream_t stream) {
  const int R = d->num_reqs;
  const int T = R > 0 ? d->cu_q_lens_host[R] : 0;
  std::vector<int32_t> bt, ctx, cu, qp;
  hipError_t e;
  if ((e = fetch_i32(ctx, context_lens, (size_t)R, stream)) != hipSuccess ||
      (e = fetch_i32(cu, cu_q_lens, (size_t)R + 1, stream)) != hipSuccess ||
      (e = fetch_i32(bt, block_tables, (size_t)R * d->block_table_stride, stream)) != hipSuccess ||
      (q_pos && (e = fetch_i32(qp, q_pos, (size_t)T, stream)) != hipSuccess))
    return hip_fail(e, "debug validation: reading the batch metadata");
  for (int r = 0; r < R; ++r)
    if (ctx[r] != d->context_lens_host[r])
      return fail(PENSIEVE_ERR_INVALID_ARG, "PENSIEVE_DEBUG: context_lens[%d] = %d on the device, %d in the host copy", r,
                  ctx[r], d->context_lens_host[r]);
  for (int r = 0; r <= R; ++r)
    if (cu[r] != d->cu_q_lens_host[r])
      return fail(PENSIEVE_ERR_INVALID_ARG, "PENSIEVE_DEBUG: cu_q_lens[%d] = %d on the device, %d in the host copy", r,
                  cu[r], d->cu_q_lens_host[r]);
  for (int r = 0; r < R; ++r) {
    const int L = ctx[r];
    const int nblk = (L + kBlockSize - 1) / kBlockSize;
    for (int j = 0; j < nblk; ++j) {
      const int32_t b = bt[(size_t)r * d->block_table_stride + j];
      if (b < 0 || b >= d->num_blocks)
        return fail(PENSIEVE_ERR_INVALID_ARG, "PENSIEVE_DEBUG: block_tables[%d][%d] = %d is outside the pool (%d blocks)",
                    r, j, b, d->num_blocks);
    }
    if (!q_pos) continue;
    for (int i = cu[r]; i < cu[r + 1]; ++i) {
      if (qp[i] < 0 || qp[i] >= L)
        return fail(PENSIEVE_ERR_INVALID_ARG, "PENSIEVE_DEBUG: q_pos[%d] = %d is outside [0, %d) of request %d", i, qp[i],
                    L, r);
      if (i > cu[r] && qp[i] <= qp[i - 1])
        return fail(PENSIEVE_ERR_INVALID_ARG, "PENSIEVE_DEBUG: q_pos is not strictly increasing at row %d (request %d)",
                    i, r);
    }
  }
  return PENSIEVE_OK;
}

}  // namespace

namespace pk {
pensieve_status set_error(pensieve_status s, const char* msg) {
  g_last_error = msg;
  return s;
}
pensieve_status clear_error() { return ok(); }
}  // namespace pk

extern "C" {

pensieve_status pensieve_kv_swap_out(void* k_pool, void* v_pool, int32_t num_blocks, void* k_host, void* v_host,
                                     int32_t num_host_blocks, const int32_t* device_blocks_host,
                                     const int32_t* host_blocks_host, int32_t n, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t dtype, void* stream) {
  return kv_swap(true, k_pool, v_pool, num_blocks, k_host, v_host, num_host_blocks, device_blocks_host,
                 host_blocks_host, n, num_kv_heads, head_dim, dtype, stream);
}

pensieve_status pensieve_kv_swap_in(void* k_pool, void* v_pool, int32_t num_blocks, void* k_host, void* v_host,
                                    int32_t num_host_blocks, const int32_t* host_blocks_host,
                                    const int32_t* device_blocks_host, int32_t n, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t dtype, void* stream) {
  return kv_swap(false, k_pool, v_pool, num_blocks, k_host, v_host, num_host_blocks, host_blocks_host,
                 device_blocks_host, n, num_kv_heads, head_dim, dtype, stream);
}


const char* pensieve_version(void) { return "pensieve 0.1 gfx950"; }

const char* pensieve_last_error(void) { return g_last_error.c_str(); }

pensieve_status pensieve_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                   const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                                   void* stream) {
  if (num_tokens < 0) return fail(PENSIEVE_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_kv_heads <= 0) return fail(PENSIEVE_ERR_INVALID_ARG, "num_kv_heads must be > 0");
  if (head_dim != 64 && head_dim != 128) return fail(PENSIEVE_ERR_UNSUPPORTED, "head_dim %d unsupported", head_dim);
  if (block_size != kBlockSize) return fail(PENSIEVE_ERR_UNSUPPORTED, "block_size %d unsupported", block_size);
  if (!valid_dtype(dtype)) return fail(PENSIEVE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (num_blocks <= 0) return fail(PENSIEVE_ERR_INVALID_ARG, "num_blocks must be > 0");
  if (num_kv_heads > 65535) return fail(PENSIEVE_ERR_UNSUPPORTED, "num_kv_heads > 65535");
  if (num_tokens == 0) return ok();
  if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping)
    return fail(PENSIEVE_ERR_INVALID_ARG, "a device pointer is NULL");
  if (debug_validation()) {
    const pensieve_status s = validate_slots(slot_mapping, num_tokens, num_blocks, static_cast<hipStream_t>(stream));
    if (s != PENSIEVE_OK) return s;
  }
  TraceScope trace(kTraceAppend, num_tokens, static_cast<hipStream_t>(stream));
  hipError_t e = pk::launch_kv_append(k_new, v_new, k_pool, v_pool, slot_mapping, num_tokens, num_kv_heads, head_dim,
                                      elem_bytes(dtype), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  return ok();
}

pensieve_status pensieve_kv_append_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                       const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t src_dtype,
                                       float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0) return fail(PENSIEVE_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_kv_heads <= 0) return fail(PENSIEVE_ERR_INVALID_ARG, "num_kv_heads must be > 0");
  if (head_dim != 64 && head_dim != 128) return fail(PENSIEVE_ERR_UNSUPPORTED, "head_dim %d unsupported", head_dim);
  if (block_size != kBlockSize) return fail(PENSIEVE_ERR_UNSUPPORTED, "block_size %d unsupported", block_size);
  if (src_dtype != PENSIEVE_F16 && src_dtype != PENSIEVE_BF16)
    return fail(PENSIEVE_ERR_UNSUPPORTED, "src_dtype %d unsupported (F16 or BF16)", src_dtype);
  if (!valid_scale(k_scale) || !valid_scale(v_scale))
    return fail(PENSIEVE_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  if (num_blocks <= 0) return fail(PENSIEVE_ERR_INVALID_ARG, "num_blocks must be > 0");
  if (num_kv_heads > 65535) return fail(PENSIEVE_ERR_UNSUPPORTED, "num_kv_heads > 65535");
  if (num_tokens == 0) return ok();
  if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping)
    return fail(PENSIEVE_ERR_INVALID_ARG, "a device pointer is NULL");
  if (debug_validation()) {
    const pensieve_status s = validate_slots(slot_mapping, num_tokens, num_blocks, static_cast<hipStream_t>(stream));
    if (s != PENSIEVE_OK) return s;
  }
  TraceScope trace(kTraceAppend, num_tokens, static_cast<hipStream_t>(stream));
  hipError_t e = pk::launch_kv_append_fp8(k_new, v_new, k_pool, v_pool, slot_mapping, num_tokens, num_kv_heads,
                                          head_dim, src_dtype, k_scale, v_scale, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv_append_fp8 launch");
  return ok();
}

pensieve_status pensieve_attn_workspace_size(const pensieve_batch_desc* desc, int32_t num_partitions, size_t* bytes) {
  pensieve_status s = check_desc(desc);
  if (s != PENSIEVE_OK) return s;
  if (!bytes) return fail(PENSIEVE_ERR_INVALID_ARG, "bytes is NULL");
  if (num_partitions < 0 || num_partitions > kMaxPartitions)
    return fail(PENSIEVE_ERR_INVALID_ARG, "num_partitions must be in [0, %d]", kMaxPartitions);
  thread_local Plan plan;   // keeps its capacity from call to call
  build_plan(desc, num_partitions, plan);
  *bytes = plan.bytes();
  return ok();
}

pensieve_status pensieve_attn_fwd(const pensieve_batch_desc* desc, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* cu_q_lens, const int32_t* q_pos, void* o, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  pensieve_status s = check_desc(desc);
  if (s != PENSIEVE_OK) return s;
  if ((s = check_attn_pointers(desc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens)) != PENSIEVE_OK) return s;
  if (total_q(desc) == 0) return ok();
  if (!o) return fail(PENSIEVE_ERR_INVALID_ARG, "o is NULL");
  if (o == q) return fail(PENSIEVE_ERR_INVALID_ARG, "o must not alias q");
  if ((s = refuse_capture(static_cast<hipStream_t>(stream))) != PENSIEVE_OK) return s;
  if (debug_validation() &&
      (s = validate_batch(desc, block_tables, context_lens, cu_q_lens, q_pos, static_cast<hipStream_t>(stream))) !=
          PENSIEVE_OK)
    return s;
  thread_local Plan plan;   // keeps its capacity from call to call
  build_plan(desc, 0, plan);
  if (!workspace || workspace_bytes < plan.bytes())
    return fail(PENSIEVE_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", plan.bytes(),
                workspace ? workspace_bytes : (size_t)0);
  pk::AttnArgs a = make_args(desc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos);
  a.o = static_cast<uint8_t*>(o);
  a.write_partials = 0;
  a.part_stride = 1;
  return run_plan(desc, plan, a, workspace, static_cast<hipStream_t>(stream));
}

pensieve_status pensieve_attn_fwd_noalloc(const pensieve_batch_desc* desc, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_tables, const int32_t* context_lens,
                                          const int32_t* cu_q_lens, const int32_t* q_pos, void* o, void* stream) {
  pensieve_status s = check_desc(desc);
  if (s != PENSIEVE_OK) return s;
  if ((s = check_attn_pointers(desc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens)) != PENSIEVE_OK) return s;
  if (total_q(desc) == 0) return ok();
  if (!o) return fail(PENSIEVE_ERR_INVALID_ARG, "o is NULL");
  if (o == q) return fail(PENSIEVE_ERR_INVALID_ARG, "o must not alias q");
  if ((s = refuse_capture(static_cast<hipStream_t>(stream))) != PENSIEVE_OK) return s;
  if (debug_validation() &&
      (s = validate_batch(desc, block_tables, context_lens, cu_q_lens, q_pos, static_cast<hipStream_t>(stream))) !=
          PENSIEVE_OK)
    return s;
  thread_local Plan plan;   // keeps its capacity from call to call
  build_plan(desc, 0, plan);
  if (plan.bytes() > pk::kScratchBytes)
    return fail(PENSIEVE_ERR_WORKSPACE_TOO_SMALL, "the batch needs %zu bytes of scratch; the library's scratch holds %zu",
                plan.bytes(), pk::kScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = pk::scratch_for_current_device(&scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  pk::AttnArgs a = make_args(desc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos);
  a.o = static_cast<uint8_t*>(o);
  a.write_partials = 0;
  a.part_stride = 1;
  return run_plan(desc, plan, a, scratch, static_cast<hipStream_t>(stream), Upload::kPageable);
}

pensieve_status pensieve_attn_split_partial(const pensieve_batch_desc* desc, int32_t num_partitions, const void* q,
                                            const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                            const int32_t* context_lens, const int32_t* cu_q_lens,
                                            const int32_t* q_pos, float* part_o, float* part_m, float* part_l,
                                            void* workspace, size_t workspace_bytes, void* stream) {
  pensieve_status s = check_desc(desc);
  if (s != PENSIEVE_OK) return s;
  if (num_partitions < 1 || num_partitions > kMaxPartitions)
    return fail(PENSIEVE_ERR_INVALID_ARG, "num_partitions must be in [1, %d]", kMaxPartitions);
  if ((s = check_attn_pointers(desc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens)) != PENSIEVE_OK) return s;
  if (total_q(desc) == 0) return ok();
  if (!part_o || !part_m || !part_l) return fail(PENSIEVE_ERR_INVALID_ARG, "a partial buffer is NULL");
  if ((s = refuse_capture(static_cast<hipStream_t>(stream))) != PENSIEVE_OK) return s;
  if (debug_validation() &&
      (s = validate_batch(desc, block_tables, context_lens, cu_q_lens, q_pos, static_cast<hipStream_t>(stream))) !=
          PENSIEVE_OK)
    return s;
  thread_local Plan plan;   // keeps its capacity from call to call
  build_plan(desc, num_partitions, plan);
  if (!workspace || workspace_bytes < plan.bytes())
    return fail(PENSIEVE_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", plan.bytes(),
                workspace ? workspace_bytes : (size_t)0);
  pk::AttnArgs a = make_args(desc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos);
  a.part_o = part_o;
  a.part_m = part_m;
  a.part_l = part_l;
  a.part_stride = num_partitions;
  a.write_partials = 1;
  return run_plan(desc, plan, a, workspace, static_cast<hipStream_t>(stream));
}

pensieve_status pensieve_attn_split_merge(const float* part_o, const float* part_m, const float* part_l,
                                          int32_t total_rows, int32_t num_heads, int32_t head_dim,
                                          int32_t num_partitions, int32_t dtype, void* o, void* stream) {
  if (total_rows < 0 || num_heads <= 0) return fail(PENSIEVE_ERR_INVALID_ARG, "bad total_q / num_heads");
  if (head_dim != 64 && head_dim != 128) return fail(PENSIEVE_ERR_UNSUPPORTED, "head_dim %d unsupported", head_dim);
  if (num_partitions < 1 || num_partitions > kMaxPartitions)
    return fail(PENSIEVE_ERR_INVALID_ARG, "num_partitions must be in [1, %d]", kMaxPartitions);
  if (!valid_dtype(dtype)) return fail(PENSIEVE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  const long long rows = (long long)total_rows * num_heads;
  if (rows == 0) return ok();
  if (rows > (1LL << 31) - 4) return fail(PENSIEVE_ERR_UNSUPPORTED, "too many rows");
  if (!part_o || !part_m || !part_l || !o) return fail(PENSIEVE_ERR_INVALID_ARG, "a pointer is NULL");
  TraceScope trace(kTraceMerge, (int)rows, static_cast<hipStream_t>(stream));
  hipError_t e = pk::launch_split_merge(part_o, part_m, part_l, (int)rows, num_heads, head_dim, num_partitions, nullptr,
                                        dtype, o, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "split merge launch");
  return ok();
}

pensieve_status pensieve_debug_plan(const pensieve_batch_desc* desc, int32_t num_partitions, int32_t* items_host,
                                    int32_t max_items, int32_t* num_items) {
  pensieve_status s = check_desc(desc);
  if (s != PENSIEVE_OK) return s;
  if (num_partitions < 0 || num_partitions > kMaxPartitions)
    return fail(PENSIEVE_ERR_INVALID_ARG, "num_partitions must be in [0, %d]", kMaxPartitions);
  if (!num_items || (max_items > 0 && !items_host)) return fail(PENSIEVE_ERR_INVALID_ARG, "NULL output");
  thread_local Plan plan;   // keeps its capacity from call to call
  build_plan(desc, num_partitions, plan);
  *num_items = (int32_t)plan.planned.size();
  for (int i = 0; i < (int)plan.planned.size() && i < max_items; ++i) {
    const PlannedItem& p = plan.planned[i];
    int32_t* o = items_host + 10 * i;
    o[0] = p.kernel;
    o[1] = p.w.req;
    o[2] = p.w.kv_head;
    o[3] = p.w.q_begin;
    o[4] = p.w.q_count;
    o[5] = p.w.part;
    o[6] = p.w.num_parts;
    o[7] = (int32_t)std::min<long long>(p.cost, 0x7fffffff);
    o[8] = p.w.head_begin;
    o[9] = p.w.head_count;
  }
  return ok();
}

pensieve_status pensieve_trace_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_trace_mu);
  g_trace_on = enable > 0;
  g_trace_every = enable > 0 ? enable : 1;
  for (long long& n : g_trace_seen) n = 0;
  // Warm the event pool now, so that a timed loop traced from here on creates none.
  while (g_trace_on && g_event_pool.size() < kTracePoolWarm) {
    hipEvent_t e = nullptr;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return hip_fail(err, "trace event pool");
    g_event_pool.push_back(e);
  }
  return ok();
}

pensieve_status pensieve_trace_read(pensieve_trace_record* records_host, int32_t max_records, int32_t* num_records) {
  if (!num_records || (max_records > 0 && !records_host)) return fail(PENSIEVE_ERR_INVALID_ARG, "NULL output");
  std::lock_guard<std::mutex> lk(g_trace_mu);
  while (!g_pending.empty()) {
    const hipError_t e = hipEventSynchronize(g_pending.front().stop);
    if (e != hipSuccess && g_trace_error == hipSuccess) g_trace_error = e;
    finish_entry(g_pending.front());
    g_pending.pop_front();
  }
  const int32_t n = (int32_t)std::min<size_t>(g_records.size(), (size_t)std::max(0, max_records));
  if (n > 0) std::memcpy(records_host, g_records.data(), n * sizeof(pensieve_trace_record));
  g_records.clear();
  *num_records = n;
  const hipError_t err = g_trace_error;
  g_trace_error = hipSuccess;
  if (err != hipSuccess) return hip_fail(err, "trace read");
  return ok();
}

}  // extern "C"
