// Host batch planner for chunked SGMV LoRA.
//
// Follows the chunked_backend.py page (class ChunkedSgmvLoRABackend):
//  - chunk size: _determine_chunk_size / _determine_chunk_size_for_tokens;
//  - permutation: _get_permutation sorts tokens by their request's adapter
//    slot with a stable sort.  A stable counting sort by slot produces the
//    identical array in O(s + L) instead of O(s log s);
//  - segments: _get_segments_info cuts each run of equal slots into pieces of
//    `chunk` tokens, remainder last, ascending by slot;
//  - request boundaries: _build_req_seg_indptr;
//  - padding of unused segment entries: the graph branch of
//    prepare_lora_batch (slot 0, boundary repeated = zero length).
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "sgg_internal.h"
#include "../../include/sgg_lora.h"

namespace sgg {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SGG_OK;
}

static int32_t chunk_for_tokens(int64_t n, int32_t max_chunk) {
  if (max_chunk <= SGG_MIN_CHUNK_SIZE) return SGG_MIN_CHUNK_SIZE;
  int32_t wanted = n >= 256 ? 128 : (n >= 64 ? 32 : 16);
  return wanted < max_chunk ? wanted : max_chunk;
}

}  // namespace sgg

extern "C" const char* lora_last_error(void) { return sgg::g_last_error.c_str(); }

extern "C" int64_t lora_plan_max_segments(int64_t num_tokens, int32_t max_loras,
                                          int32_t min_chunk) {
  if (num_tokens <= 0) return 0;
  if (min_chunk < 1) min_chunk = 1;
  int64_t by_chunks = (num_tokens + min_chunk - 1) / min_chunk + (max_loras > 0 ? max_loras : 0);
  return by_chunks < num_tokens ? by_chunks : num_tokens;
}

extern "C" int lora_plan_segments(const int32_t* seq_lens, const int32_t* req_slots,
                                  int32_t num_reqs, int32_t max_loras, int32_t is_decode,
                                  int32_t max_chunk_size, int32_t chunk_size_override,
                                  int32_t* permutation, int64_t perm_capacity,
                                  int32_t* seg_indptr, int32_t* seg_slots, int32_t seg_capacity,
                                  int32_t* req_seg_indptr, int32_t* out_num_segments,
                                  int32_t* out_chunk_size, int64_t* out_num_tokens) {
  using sgg::fail;
  if (num_reqs < 0) return fail(SGG_ERR_INVALID, "num_reqs=%d is negative", num_reqs);
  if (max_loras <= 0) return fail(SGG_ERR_INVALID, "max_loras=%d must be positive", max_loras);
  if (num_reqs > 0 && req_slots == nullptr) return fail(SGG_ERR_INVALID, "req_slots is NULL");
  if (!is_decode && num_reqs > 0 && seq_lens == nullptr)
    return fail(SGG_ERR_INVALID, "seq_lens is NULL in extend mode");
  if (chunk_size_override < 0)
    return fail(SGG_ERR_INVALID, "chunk_size_override=%d is negative", chunk_size_override);
  if (seg_capacity < 0) return fail(SGG_ERR_INVALID, "seg_capacity=%d is negative", seg_capacity);
  if (seg_indptr == nullptr || (seg_capacity > 0 && seg_slots == nullptr))
    return fail(SGG_ERR_INVALID, "seg_indptr / seg_slots is NULL");

  // Tokens per slot; validate lengths and slots.
  std::vector<int64_t> count(static_cast<size_t>(max_loras), 0);
  int64_t s = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    int32_t len = seq_lens ? seq_lens[r] : 1;
    if (len < 0) return fail(SGG_ERR_INVALID, "seq_lens[%d]=%d is negative", r, len);
    if (is_decode && len != 1)
      return fail(SGG_ERR_INVALID, "decode mode needs one token per request (seq_lens[%d]=%d)",
                  r, len);
    int32_t a = req_slots[r];
    if (a < 0 || a >= max_loras)
      return fail(SGG_ERR_CAPACITY, "req_slots[%d]=%d outside [0, %d)", r, a, max_loras);
    count[a] += len;
    s += len;
  }
  if (s > INT32_MAX) return fail(SGG_ERR_INVALID, "%lld tokens exceed int32 indexing",
                                 static_cast<long long>(s));
  if (s > 0 && permutation == nullptr) return fail(SGG_ERR_INVALID, "permutation is NULL");
  if (perm_capacity < s)
    return fail(SGG_ERR_CAPACITY, "permutation capacity %lld < %lld tokens",
                static_cast<long long>(perm_capacity), static_cast<long long>(s));

  const int32_t chunk = chunk_size_override > 0
                            ? chunk_size_override
                            : sgg::chunk_for_tokens(is_decode ? num_reqs : s, max_chunk_size);

  int64_t n_seg = 0;
  for (int32_t a = 0; a < max_loras; ++a) n_seg += (count[a] + chunk - 1) / chunk;
  if (n_seg > seg_capacity)
    return fail(SGG_ERR_CAPACITY, "plan needs %lld segments, capacity is %d",
                static_cast<long long>(n_seg), seg_capacity);

  // Stable counting sort: slot a's tokens start at the sum of smaller slots'
  // counts and keep their original order.
  std::vector<int64_t> next(static_cast<size_t>(max_loras), 0);
  int64_t acc = 0;
  for (int32_t a = 0; a < max_loras; ++a) {
    next[a] = acc;
    acc += count[a];
  }
  int64_t t = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    int32_t len = seq_lens ? seq_lens[r] : 1;
    int64_t& pos = next[req_slots[r]];
    for (int32_t i = 0; i < len; ++i) permutation[pos++] = static_cast<int32_t>(t++);
  }

  // Segments: runs in ascending slot order, full chunks then the remainder.
  int64_t i = 0, start = 0;
  seg_indptr[0] = 0;
  for (int32_t a = 0; a < max_loras; ++a) {
    int64_t left = count[a];
    while (left > 0) {
      int64_t len = left < chunk ? left : chunk;
      seg_slots[i] = a;
      start += len;
      seg_indptr[i + 1] = static_cast<int32_t>(start);
      ++i;
      left -= len;
    }
  }
  for (; i < seg_capacity; ++i) {
    seg_slots[i] = 0;
    seg_indptr[i + 1] = static_cast<int32_t>(s);
  }

  if (req_seg_indptr) {
    int64_t c = 0;
    req_seg_indptr[0] = 0;
    for (int32_t r = 0; r < num_reqs; ++r) {
      c += seq_lens ? seq_lens[r] : 1;
      req_seg_indptr[r + 1] = static_cast<int32_t>(c);
    }
  }
  if (out_num_segments) *out_num_segments = static_cast<int32_t>(n_seg);
  if (out_chunk_size) *out_chunk_size = chunk;
  if (out_num_tokens) *out_num_tokens = s;
  return sgg::ok();
}

// Plan of a pruned lm_head pass (chunked_backend.py page:
// _prepare_lm_head_batch_info, _build_lm_head_batch_info).  The pruned tokens
// stay in original order (identity permutation).  Segments come from the
// page's merge_and_chunk_segments, which it imports but does not print; the
// plain reading is taken: requests with no pruned token are dropped,
// consecutive requests of one slot form a run, and each run is cut into
// pieces of `chunk` tokens, remainder last.  The chunk follows the
// token-count rule over the pruned total.
extern "C" int lora_plan_lm_head(const int32_t* pruned_lens, const int32_t* req_slots,
                                 int32_t num_reqs, int32_t max_loras, int32_t max_chunk_size,
                                 int32_t chunk_size_override, int32_t* permutation,
                                 int64_t perm_capacity, int32_t* seg_indptr, int32_t* seg_slots,
                                 int32_t seg_capacity, int32_t* out_num_segments,
                                 int32_t* out_chunk_size, int64_t* out_num_tokens) {
  using sgg::fail;
  if (num_reqs < 0) return fail(SGG_ERR_INVALID, "num_reqs=%d is negative", num_reqs);
  if (max_loras <= 0) return fail(SGG_ERR_INVALID, "max_loras=%d must be positive", max_loras);
  if (num_reqs > 0 && (req_slots == nullptr || pruned_lens == nullptr))
    return fail(SGG_ERR_INVALID, "pruned_lens or req_slots is NULL");
  if (chunk_size_override < 0)
    return fail(SGG_ERR_INVALID, "chunk_size_override=%d is negative", chunk_size_override);
  if (seg_capacity < 0) return fail(SGG_ERR_INVALID, "seg_capacity=%d is negative", seg_capacity);
  if (seg_indptr == nullptr || (seg_capacity > 0 && seg_slots == nullptr))
    return fail(SGG_ERR_INVALID, "seg_indptr / seg_slots is NULL");

  int64_t s = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    if (pruned_lens[r] < 0)
      return fail(SGG_ERR_INVALID, "pruned_lens[%d]=%d is negative", r, pruned_lens[r]);
    if (req_slots[r] < 0 || req_slots[r] >= max_loras)
      return fail(SGG_ERR_CAPACITY, "req_slots[%d]=%d outside [0, %d)", r, req_slots[r],
                  max_loras);
    s += pruned_lens[r];
  }
  if (s > INT32_MAX) return fail(SGG_ERR_INVALID, "%lld tokens exceed int32 indexing",
                                 static_cast<long long>(s));
  if (s > 0 && permutation == nullptr) return fail(SGG_ERR_INVALID, "permutation is NULL");
  if (perm_capacity < s)
    return fail(SGG_ERR_CAPACITY, "permutation capacity %lld < %lld tokens",
                static_cast<long long>(perm_capacity), static_cast<long long>(s));
  const int32_t chunk = chunk_size_override > 0 ? chunk_size_override
                                                : sgg::chunk_for_tokens(s, max_chunk_size);

  // count the segments first (runs of one slot, chunked)
  int64_t n_seg = 0;
  for (int32_t r = 0; r < num_reqs;) {
    if (pruned_lens[r] == 0) { ++r; continue; }
    const int32_t slot = req_slots[r];
    int64_t run = 0;
    while (r < num_reqs && (pruned_lens[r] == 0 || req_slots[r] == slot)) run += pruned_lens[r++];
    n_seg += (run + chunk - 1) / chunk;
  }
  if (n_seg > seg_capacity)
    return fail(SGG_ERR_CAPACITY, "plan needs %lld segments, capacity is %d",
                static_cast<long long>(n_seg), seg_capacity);

  for (int64_t t = 0; t < s; ++t) permutation[t] = static_cast<int32_t>(t);
  int64_t i = 0, start = 0;
  seg_indptr[0] = 0;
  for (int32_t r = 0; r < num_reqs;) {
    if (pruned_lens[r] == 0) { ++r; continue; }
    const int32_t slot = req_slots[r];
    int64_t run = 0;
    while (r < num_reqs && (pruned_lens[r] == 0 || req_slots[r] == slot)) run += pruned_lens[r++];
    while (run > 0) {
      const int64_t len = run < chunk ? run : chunk;
      seg_slots[i] = slot;
      start += len;
      seg_indptr[i + 1] = static_cast<int32_t>(start);
      ++i;
      run -= len;
    }
  }
  for (; i < seg_capacity; ++i) {
    seg_slots[i] = 0;
    seg_indptr[i + 1] = static_cast<int32_t>(s);
  }
  if (out_num_segments) *out_num_segments = static_cast<int32_t>(n_seg);
  if (out_chunk_size) *out_chunk_size = chunk;
  if (out_num_tokens) *out_num_tokens = s;
  return sgg::ok();
}
