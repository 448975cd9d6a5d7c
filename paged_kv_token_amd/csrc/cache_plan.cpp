// Host-side cache planning for one serving step ("Stateful Large Language Model Serving with
// Pensieve", Methodology: cached KV is dropped at block granularity, weighing how active a
// conversation is and what its tokens cost to recompute; dropped tokens are recomputed together
// with the conversation's next turn, over a cache that is then partly refreshed and scattered).
//
// Eviction drops the leading resident block of some unscheduled conversation, one block at a
// time, always the one whose loss costs least: activity x (block index + 1), the second factor
// being the context, in blocks, that a recomputation of that block attends over.  A
// conversation's leading blocks are therefore its cheapest, and idle conversations the cheapest
// overall.  The batch builder turns every scheduled conversation into one request whose query
// rows are its dropped leading tokens (recompute) followed by its new tokens, and gives it the
// positions, context length, fresh blocks and append slots that kv_append and the attention
// call need.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <queue>
#include <utility>
#include <vector>

#include "host_status.h"
#include "pensieve.h"

namespace {

constexpr int kBlock = 16;

int64_t blocks_for(int64_t tokens) { return (tokens + kBlock - 1) / kBlock; }

pensieve_status bad(const char* what) { return pk::set_error(PENSIEVE_ERR_INVALID_ARG, what); }

pensieve_status check_convs(const pensieve_conversation* convs, int32_t n) {
  if (n < 0) return bad("n < 0");
  if (n > 0 && !convs) return bad("conversations is NULL");
  for (int32_t c = 0; c < n; ++c) {
    const pensieve_conversation& v = convs[c];
    if (v.cached_tokens < 0 || v.new_tokens < 0) return bad("negative token count");
    if ((int64_t)v.cached_tokens + v.new_tokens > 0x7fffffff) return bad("conversation longer than 2^31-1 tokens");
    if (v.dropped_blocks < 0 || v.dropped_blocks > blocks_for(v.cached_tokens))
      return bad("dropped_blocks outside the conversation's cached blocks");
    if (!std::isfinite(v.activity) || v.activity < 0.f) return bad("activity must be finite and >= 0");
  }
  return PENSIEVE_OK;
}

// Fresh blocks a scheduled conversation takes this step: the dropped blocks it recomputes plus
// the logical blocks its new tokens open.
int64_t step_blocks(const pensieve_conversation& v) {
  return v.dropped_blocks + blocks_for((int64_t)v.cached_tokens + v.new_tokens) - blocks_for(v.cached_tokens);
}

// Recompute rows of a scheduled conversation: every position of its dropped blocks.
int64_t recompute_rows(const pensieve_conversation& v) {
  return std::min<int64_t>((int64_t)kBlock * v.dropped_blocks, v.cached_tokens);
}

}  // namespace

extern "C" {

pensieve_status pensieve_cache_plan_evictions(const pensieve_conversation* conversations, int32_t n,
                                              int32_t free_blocks, int32_t* evict_blocks_host,
                                              int32_t* freed_blocks) {
  pensieve_status s = check_convs(conversations, n);
  if (s != PENSIEVE_OK) return s;
  if (free_blocks < 0) return bad("free_blocks < 0");
  if (n > 0 && !evict_blocks_host) return bad("evict_blocks_host is NULL");
  if (!freed_blocks) return bad("freed_blocks is NULL");
  int64_t need = 0;
  for (int32_t c = 0; c < n; ++c) {
    evict_blocks_host[c] = 0;
    if (conversations[c].new_tokens > 0) need += step_blocks(conversations[c]);
  }
  *freed_blocks = 0;
  if (need <= free_blocks) return pk::clear_error();
  // Min-heap of (cost of dropping it, conversation) over the next leading resident block of
  // every unscheduled conversation that still has one; ties go to the lower conversation index.
  typedef std::pair<double, int32_t> Entry;
  std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> heap;
  auto offer = [&](int32_t c) {
    const pensieve_conversation& v = conversations[c];
    const int64_t next = (int64_t)v.dropped_blocks + evict_blocks_host[c];
    if (next < blocks_for(v.cached_tokens)) heap.push(Entry((double)v.activity * (double)(next + 1), c));
  };
  for (int32_t c = 0; c < n; ++c)
    if (conversations[c].new_tokens == 0) offer(c);
  int64_t freed = 0;
  while (free_blocks + freed < need && !heap.empty()) {
    const int32_t c = heap.top().second;
    heap.pop();
    ++evict_blocks_host[c];
    ++freed;
    offer(c);
  }
  *freed_blocks = (int32_t)freed;
  if (free_blocks + freed < need)
    return pk::set_error(PENSIEVE_ERR_UNSUPPORTED,
                         "the step does not fit even with every block of the unscheduled conversations dropped");
  return pk::clear_error();
}

pensieve_status pensieve_cache_build_batch(const pensieve_conversation* conversations, int32_t n,
                                           int32_t* block_tables_host, int32_t block_table_stride,
                                           const int32_t* free_list_host, int32_t free_count, int32_t max_rows,
                                           int32_t* num_reqs, int32_t* total_rows, int32_t* blocks_used,
                                           int32_t* request_conv_host, int32_t* cu_q_lens_host,
                                           int32_t* context_lens_host, int32_t* q_pos_host,
                                           int32_t* slot_mapping_host, int32_t* req_block_tables_host) {
  pensieve_status s = check_convs(conversations, n);
  if (s != PENSIEVE_OK) return s;
  if (!num_reqs || !total_rows || !blocks_used) return bad("a count output is NULL");
  if (block_table_stride < 0) return bad("block_table_stride < 0");
  int64_t rows = 0, blocks = 0;
  int32_t reqs = 0;
  for (int32_t c = 0; c < n; ++c) {
    const pensieve_conversation& v = conversations[c];
    if (v.new_tokens == 0) continue;
    if (blocks_for((int64_t)v.cached_tokens + v.new_tokens) > block_table_stride)
      return bad("a scheduled conversation needs more blocks than block_table_stride");
    rows += recompute_rows(v) + v.new_tokens;
    blocks += step_blocks(v);
    ++reqs;
  }
  if (rows > 0x7fffffff || blocks > 0x7fffffff) return bad("batch too large");
  *num_reqs = reqs;
  *total_rows = (int32_t)rows;
  *blocks_used = (int32_t)blocks;
  if (max_rows < 0) return pk::clear_error();  // sizes only
  if (rows > max_rows) return bad("max_rows is smaller than the batch");
  if (blocks > free_count) return bad("free_list_host holds fewer blocks than the batch takes");
  if (!cu_q_lens_host) return bad("cu_q_lens_host is NULL");
  if (reqs > 0 && (!block_tables_host || !free_list_host || !request_conv_host || !context_lens_host ||
                   !slot_mapping_host || !q_pos_host || !req_block_tables_host))
    return bad("an array argument is NULL");
  int32_t r = 0, row = 0, next_free = 0;
  cu_q_lens_host[0] = 0;
  for (int32_t c = 0; c < n; ++c) {
    const pensieve_conversation& v = conversations[c];
    if (v.new_tokens == 0) continue;
    int32_t* bt = block_tables_host + (size_t)c * block_table_stride;
    // Fresh blocks: first the dropped leading blocks, then the logical blocks the new tokens open.
    for (int32_t j = 0; j < v.dropped_blocks; ++j) bt[j] = free_list_host[next_free++];
    const int32_t opened_from = (int32_t)blocks_for(v.cached_tokens);
    const int32_t opened_to = (int32_t)blocks_for((int64_t)v.cached_tokens + v.new_tokens);
    for (int32_t j = opened_from; j < opened_to; ++j) bt[j] = free_list_host[next_free++];
    auto emit = [&](int32_t pos) {
      q_pos_host[row] = pos;
      slot_mapping_host[row] = bt[pos / kBlock] * kBlock + pos % kBlock;
      ++row;
    };
    const int32_t rec = (int32_t)recompute_rows(v);
    for (int32_t p = 0; p < rec; ++p) emit(p);
    for (int32_t p = 0; p < v.new_tokens; ++p) emit(v.cached_tokens + p);
    request_conv_host[r] = c;
    context_lens_host[r] = v.cached_tokens + v.new_tokens;
    if (block_table_stride > 0)
      std::memcpy(req_block_tables_host + (size_t)r * block_table_stride, bt, sizeof(int32_t) * block_table_stride);
    cu_q_lens_host[r + 1] = row;
    ++r;
  }
  return pk::clear_error();
}

}  // extern "C"
