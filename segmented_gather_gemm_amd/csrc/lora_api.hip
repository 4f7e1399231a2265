// C-ABI device entry points: argument validation (host only, before anything
// is enqueued), tile choice and kernel launches.
#include <atomic>
#include <cinttypes>
#include <cstring>
#include <mutex>
#include <vector>

#include "sgg_internal.h"
#include "sgg_kernels.h"
#include "../../include/sgg_lora.h"

using sgg::fail;

namespace {

// lora_set_option values.
std::atomic<int64_t> g_fused_stacked{0};
std::atomic<int64_t> g_fused_ksplit{0};
std::atomic<int64_t> g_shrink_valu{0};
std::atomic<int64_t> g_shrink_pair_tiles{0};
std::atomic<int64_t> g_fused_trace{0};          // device address of a block timeline, or 0
std::atomic<int64_t> g_fused_trace_blocks{0};
std::atomic<int64_t> g_expand_deal_tiles{1};
std::atomic<int64_t> g_spin_limit{int64_t{1} << 20};

#define SGG_CHECK(cond, code, ...) \
  do {                             \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int check_plan(int64_t s, int32_t num_segments, const int32_t* seg_indptr,
               const int32_t* seg_slots, const int32_t* permutation, const int32_t* lora_ranks,
               int32_t num_loras, int32_t chunk_size) {
  SGG_CHECK(s >= 0 && s <= INT32_MAX, SGG_ERR_INVALID, "s=%" PRId64 " outside [0, 2^31)", s);
  SGG_CHECK(num_segments >= 0, SGG_ERR_INVALID, "num_segments=%d is negative", num_segments);
  SGG_CHECK(num_loras > 0, SGG_ERR_INVALID, "num_loras=%d must be positive", num_loras);
  SGG_CHECK(chunk_size > 0, SGG_ERR_INVALID, "chunk_size=%d must be positive", chunk_size);
  // an empty plan (no tokens or no segments) may come with NULL arrays
  SGG_CHECK((seg_indptr && seg_slots && lora_ranks) || num_segments == 0, SGG_ERR_INVALID,
            "a plan array (seg_indptr, seg_slots, lora_ranks) is NULL");
  SGG_CHECK(permutation || s == 0, SGG_ERR_INVALID, "permutation is NULL");
  return SGG_OK;
}

int check_shrink(const void* x, int64_t ldx, const void* A, const void* h, int64_t ldh,
                 int64_t s, int64_t K, int32_t num_loras, int32_t c, int32_t R) {
  SGG_CHECK(A && ((x && h) || s == 0), SGG_ERR_INVALID, "x, A or h is NULL");
  SGG_CHECK(K > 0, SGG_ERR_INVALID, "in_dim=%" PRId64 " must be positive", K);
  SGG_CHECK(c >= 1 && c <= SGG_MAX_SLICES, SGG_ERR_INVALID, "num_slices=%d outside [1, %d]", c,
            SGG_MAX_SLICES);
  SGG_CHECK(R > 0, SGG_ERR_INVALID, "R=%d must be positive", R);
  SGG_CHECK(ldx >= K, SGG_ERR_INVALID, "ldx=%" PRId64 " < in_dim=%" PRId64, ldx, K);
  SGG_CHECK(ldh >= static_cast<int64_t>(c) * R, SGG_ERR_INVALID,
            "ldh=%" PRId64 " < num_slices*R=%d", ldh, c * R);
  SGG_CHECK(K % 8 == 0 && ldx % 8 == 0 && R % 8 == 0 && ldh % 8 == 0, SGG_ERR_UNSUPPORTED,
            "in_dim, ldx, R and ldh must be multiples of 8 (got %" PRId64 ", %" PRId64
            ", %d, %" PRId64 ")", K, ldx, R, ldh);
  SGG_CHECK(sgg::aligned16(x) && sgg::aligned16(A) && sgg::aligned16(h), SGG_ERR_UNSUPPORTED,
            "x, A and h must be 16-byte aligned");
  (void)s;
  (void)num_loras;
  return SGG_OK;
}

int check_expand(const void* h, int64_t ldh, const void* B, int64_t N, const void* out,
                 int64_t ldo, int32_t R, const int32_t* offs, int32_t c, int32_t max_slice,
                 const float* scalings, int64_t s) {
  SGG_CHECK(B && scalings && (h || s == 0), SGG_ERR_INVALID, "h, B or scalings is NULL");
  SGG_CHECK(out || s == 0, SGG_ERR_INVALID,
            "base_output is NULL (pass a zero-filled tensor instead)");
  SGG_CHECK(offs, SGG_ERR_INVALID, "slice_offsets is NULL");
  SGG_CHECK(c >= 1 && c <= SGG_MAX_SLICES, SGG_ERR_INVALID, "num_slices=%d outside [1, %d]", c,
            SGG_MAX_SLICES);
  SGG_CHECK(R > 0, SGG_ERR_INVALID, "R=%d must be positive", R);
  SGG_CHECK(offs[0] == 0, SGG_ERR_INVALID, "slice_offsets[0]=%d must be 0", offs[0]);
  int32_t widest = 0;
  for (int k = 0; k < c; ++k) {
    SGG_CHECK(offs[k + 1] >= offs[k], SGG_ERR_INVALID,
              "slice_offsets must be non-decreasing (offs[%d]=%d > offs[%d]=%d)", k, offs[k],
              k + 1, offs[k + 1]);
    if (offs[k + 1] - offs[k] > widest) widest = offs[k + 1] - offs[k];
  }
  SGG_CHECK(max_slice >= widest, SGG_ERR_INVALID, "max_slice_size=%d < widest slice %d",
            max_slice, widest);
  SGG_CHECK(N >= offs[c], SGG_ERR_INVALID, "B has %" PRId64 " rows < last offset %d", N, offs[c]);
  SGG_CHECK(ldo >= offs[c], SGG_ERR_INVALID, "ldo=%" PRId64 " < last offset %d", ldo, offs[c]);
  SGG_CHECK(ldh >= static_cast<int64_t>(c) * R, SGG_ERR_INVALID,
            "ldh=%" PRId64 " < num_slices*R=%d", ldh, c * R);
  SGG_CHECK(R % 8 == 0 && ldh % 8 == 0, SGG_ERR_UNSUPPORTED,
            "R and ldh must be multiples of 8 (got %d, %" PRId64 ")", R, ldh);
  SGG_CHECK(R <= 128, SGG_ERR_UNSUPPORTED, "R=%d above 128 is not supported", R);
  SGG_CHECK(sgg::aligned16(h) && sgg::aligned16(B), SGG_ERR_UNSUPPORTED,
            "h and B must be 16-byte aligned");
  SGG_CHECK((reinterpret_cast<uintptr_t>(out) & 1u) == 0, SGG_ERR_UNSUPPORTED,
            "base_output must be 2-byte aligned");
  return SGG_OK;
}

// Columns per workgroup: 128 * pairs; 256 when that still gives at least 16
// workgroups per CU, or at least 4 when the segments average 96 tokens or
// more; else 128.  Measured: 256 wins on the 28672-wide gate_up of prefill
// (1014 -> 825 us) and of the full-layer batch (192 -> 147 us), and on
// decode-shaped qkv batches of long segments (stacked call, 8192 tokens 96.9
// -> 90.5 us, 16384 tokens 162.7 -> 146.2 us; 4096 tokens, under 4 per CU,
// 44.3 vs 45.0 us); 128 wins by 1-3 us on the 4096- and 6144-wide outputs of
// the full-layer and skewed batches (segments of 44-46 tokens on average),
// whose grids are 5-10x smaller; 512 is slower everywhere.
// Rank steps of 32.
// `pairs` > 0 forces the column tile (128 * pairs).  `deal_tiles`: column
// tiles dealt to the XCDs (expand_item_of); *tiles_per_xcd gets their count
// per XCD (0: segments dealt instead).
sgg::ExpandTiling choose_expand_tiling(const int32_t* offs, int c, int num_segments, int64_t s,
                                       int R,
                                       int32_t* tile_start, int32_t* total,
                                       int32_t* tiles_per_xcd, int pairs = 0,
                                       bool deal_tiles = false) {
  sgg::ExpandTiling t{};
  t.ks = R <= 32 ? 1 : (R <= 64 ? 2 : 4);
  t.pairs = 1;
  for (int cand : {2}) {
    int64_t tiles = 0;
    for (int k = 0; k < c; ++k) tiles += (offs[k + 1] - offs[k] + 128 * cand - 1) / (128 * cand);
    const bool long_segments = num_segments > 0 && s >= 96 * static_cast<int64_t>(num_segments);
    if (tiles * num_segments >= 4096 || (long_segments && tiles * num_segments >= 1024)) {
      t.pairs = cand;
      break;
    }
  }
  if (pairs > 0) t.pairs = pairs;
  const int tn = 128 * t.pairs;
  int32_t acc = 0;
  for (int k = 0; k < c; ++k) {
    tile_start[k] = acc;
    acc += (offs[k + 1] - offs[k] + tn - 1) / tn;
  }
  tile_start[c] = acc;
  *total = acc;
  if (deal_tiles) {
    *tiles_per_xcd = (acc + sgg::kXcdCount - 1) / sgg::kXcdCount;
    t.grid = static_cast<int64_t>(sgg::kXcdCount) * num_segments * *tiles_per_xcd;
  } else {
    *tiles_per_xcd = 0;
    t.grid = sgg::grid_for(num_segments, acc);
  }
  return t;
}

// The GEMM shrink tiles address x and each slot's A block through buffer
// resources with 32-bit byte offsets; the last K step of a ragged K reads up
// to 127 bytes past a row, so the ranges keep a margin below 2^32 (the
// hardware adds the offsets in 32 bits).
bool gemm_addressable(int64_t s, int64_t ldx, int64_t K, int64_t CR) {
  const int64_t lim = (int64_t{1} << 32) - 256;
  return ((s - 1) * ldx + K) * 2 < lim && CR * K * 2 < lim;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SGG_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return SGG_OK;
}

// The shrink tiling of a call: choose_shrink_tiling (its segment-pair tiles
// only with the "shrink_pair_tiles" option on), re-tiled for the VALU form
// when the "shrink_valu" option is on.
sgg::ShrinkTiling shrink_tiling(int64_t s, int64_t K, int CR, int num_segments, int chunk,
                                bool gemm_ok = true) {
  const bool pair_ok = g_shrink_pair_tiles.load(std::memory_order_relaxed) != 0;
  sgg::ShrinkTiling t =
      sgg::choose_shrink_tiling(s, K, CR, num_segments, chunk, gemm_ok, pair_ok);
  if (g_shrink_valu.load(std::memory_order_relaxed) != 0)
    sgg::use_valu_tiles(&t, s, num_segments, chunk);
  return t;
}

sgg::ShrinkParams shrink_params(const void* x, int64_t ldx, const void* A, void* h, int64_t ldh,
                                int64_t s, int64_t K, int32_t num_loras, int32_t c, int32_t R,
                                const int32_t* seg_indptr, const int32_t* seg_slots,
                                int32_t num_segments, const int32_t* permutation,
                                const int32_t* lora_ranks, int32_t* counters, void* partial,
                                bool partials_only, const sgg::ShrinkTiling& t) {
  sgg::ShrinkParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.A = static_cast<const uint16_t*>(A);
  p.h = static_cast<uint16_t*>(h);
  p.partial = static_cast<float*>(partial);
  p.counters = counters;
  p.counter_cap = sgg::kCounterCap;
  p.seg_indptr = seg_indptr;
  p.seg_slots = seg_slots;
  p.perm = permutation;
  p.ranks = lora_ranks;
  p.ldx = ldx;
  p.ldh = ldh;
  p.s = s;
  p.K = K;
  p.kps = t.kps;
  p.L = num_loras;
  p.R = R;
  p.CR = c * R;
  p.num_segments = num_segments;
  p.mblocks = t.mblocks;
  p.nblocks = t.nblocks;
  p.ksplit = t.ksplit;
  p.partials_only = partials_only && t.ksplit > 1 ? 1 : 0;
  p.partial_bytes = static_cast<uint32_t>(t.partial_bytes < (int64_t{1} << 32) - 256
                                              ? t.partial_bytes : 0);
  p.x_rows = s;
  p.xdiv = 1;
  return p;
}

int do_shrink(const void* x, int64_t ldx, const void* A, void* h, int64_t ldh, int64_t s,
              int64_t K, int32_t num_loras, int32_t c, int32_t R, const int32_t* seg_indptr,
              const int32_t* seg_slots, int32_t num_segments, const int32_t* permutation,
              const int32_t* lora_ranks, int32_t chunk_size, int32_t* counters,
              void* partial, int64_t partial_avail, hipStream_t stream) {
  const sgg::ShrinkTiling t = shrink_tiling(
      s, K, c * R, num_segments, chunk_size, gemm_addressable(s, ldx, K, static_cast<int64_t>(c) * R));
  if (t.ksplit > 1) {
    SGG_CHECK(counters != nullptr && partial != nullptr && partial_avail >= t.partial_bytes,
              SGG_ERR_CAPACITY, "shrink workspace too small: %" PRId64
              " partial bytes needed, %" PRId64 " available", t.partial_bytes,
              partial ? partial_avail : 0);
    SGG_CHECK(t.partial_bytes < (int64_t{1} << 32) - 256, SGG_ERR_UNSUPPORTED,
              "split-K partials of %" PRId64 " bytes exceed 32-bit offsets", t.partial_bytes);
  }
  SGG_CHECK(t.grid < (int64_t{1} << 31), SGG_ERR_UNSUPPORTED, "shrink grid too large");
  const sgg::ShrinkParams p =
      shrink_params(x, ldx, A, h, ldh, s, K, num_loras, c, R, seg_indptr, seg_slots,
                    num_segments, permutation, lora_ranks, counters, partial, false, t);
  return launch_status(sgg::launch_shrink(p, t, stream), "shrink");
}

// Expand parameters; also fills the tiling.  `hpart` (may be null): h as the
// shrink's split-K partials.
sgg::ExpandParams expand_params(const void* h, int64_t ldh, const void* B, int64_t N, void* out,
                                int64_t ldo, int64_t s, int32_t num_loras, int32_t R,
                                const int32_t* offs, int32_t c, const int32_t* seg_indptr,
                                const int32_t* seg_slots, int32_t num_segments,
                                const int32_t* permutation, const int32_t* lora_ranks,
                                const float* scalings, const float* hpart, int32_t hsplit,
                                sgg::ExpandTiling* tiling, int pairs = 0,
                                bool segment_dealing = false) {
  sgg::ExpandParams p{};
  const bool deal = !segment_dealing && g_expand_deal_tiles.load(std::memory_order_relaxed) != 0;
  *tiling = choose_expand_tiling(offs, c, num_segments, s, R, p.tile_start, &p.total_tiles,
                                 &p.tiles_per_xcd, pairs, deal);
  bool vec8 = sgg::aligned16(out) && ldo % 8 == 0;
  for (int k = 0; k <= c; ++k) {
    p.offs[k] = offs[k];
    vec8 = vec8 && offs[k] % 8 == 0;
  }
  p.h = static_cast<const uint16_t*>(h);
  p.hpart = hpart;
  p.hsplit = hpart ? hsplit : 0;
  p.ldp = static_cast<int64_t>(c) * R;
  {
    const int64_t hb = static_cast<int64_t>(p.hsplit) * s * p.ldp * 4;
    p.hpart_bytes = static_cast<uint32_t>(hb < (int64_t{1} << 32) - 256 ? hb : 0);
  }
  p.B = static_cast<const uint16_t*>(B);
  p.out = static_cast<uint16_t*>(out);
  p.seg_indptr = seg_indptr;
  p.seg_slots = seg_slots;
  p.perm = permutation;
  p.ranks = lora_ranks;
  p.scalings = scalings;
  p.ldh = ldh;
  p.ldo = ldo;
  p.s = s;
  p.N = N;
  p.L = num_loras;
  p.R = R;
  p.c = c;
  p.num_segments = num_segments;
  p.vec8 = vec8 ? 1 : 0;
  return p;
}

int do_expand(const void* h, int64_t ldh, const void* B, int64_t N, void* out, int64_t ldo,
              int64_t s, int32_t num_loras, int32_t R, const int32_t* offs, int32_t c,
              const int32_t* seg_indptr, const int32_t* seg_slots, int32_t num_segments,
              const int32_t* permutation, const int32_t* lora_ranks, const float* scalings,
              const float* hpart, int32_t hsplit, hipStream_t stream) {
  sgg::ExpandTiling t{};
  const sgg::ExpandParams p =
      expand_params(h, ldh, B, N, out, ldo, s, num_loras, R, offs, c, seg_indptr, seg_slots,
                    num_segments, permutation, lora_ranks, scalings, hpart, hsplit, &t);
  SGG_CHECK(t.grid < (int64_t{1} << 31), SGG_ERR_UNSUPPORTED, "expand grid too large");
  return launch_status(sgg::launch_expand(p, t, stream), "expand");
}

}  // namespace

extern "C" int64_t lora_shrink_workspace_bytes(int64_t s, int64_t in_dim, int32_t num_slices,
                                               int32_t R, int32_t num_segments,
                                               int32_t chunk_size) {
  if (s <= 0 || in_dim <= 0 || num_slices <= 0 || R <= 0 || num_segments <= 0 || chunk_size <= 0)
    return 0;
  const sgg::ShrinkTiling t =
      shrink_tiling(s, in_dim, num_slices * R, num_segments, chunk_size);
  return t.ksplit > 1 ? sgg::kCounterBytes + t.partial_bytes : 0;
}

extern "C" int64_t lora_qkv_workspace_bytes(int64_t s, int64_t in_dim, int32_t num_slices,
                                            int32_t R, int32_t num_segments, int32_t chunk_size) {
  if (s <= 0 || num_slices <= 0 || R <= 0) return 0;
  int64_t partial = 0;
  const int64_t CR = static_cast<int64_t>(num_slices) * R;
  if (in_dim > 0 && num_segments > 0 && chunk_size > 0) {
    const sgg::ShrinkTiling t =
        shrink_tiling(s, in_dim, static_cast<int>(CR), num_segments, chunk_size);
    partial = t.partial_bytes;
    // room for the one-launch form's partials (up to kFusedMaxSplit K ranges)
    if (t.ksplit > 1 && CR <= 48) {
      const int64_t fused = sgg::round_up(sgg::kFusedMaxSplit * s * CR * 4, 256);
      partial = fused > partial ? fused : partial;
    }
  }
  return sgg::kCounterBytes + sgg::round_up(s * CR * 2, 256) + partial;
}

extern "C" int lora_shrink(const void* x, int64_t ldx, const void* A, void* h, int64_t ldh,
                           int64_t s, int64_t in_dim, int32_t num_loras, int32_t num_slices,
                           int32_t R, const int32_t* seg_indptr, const int32_t* seg_slots,
                           int32_t num_segments, const int32_t* permutation,
                           const int32_t* lora_ranks, int32_t chunk_size, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  int rc = check_plan(s, num_segments, seg_indptr, seg_slots, permutation, lora_ranks, num_loras,
                      chunk_size);
  if (rc) return rc;
  rc = check_shrink(x, ldx, A, h, ldh, s, in_dim, num_loras, num_slices, R);
  if (rc) return rc;
  if (s == 0 || num_segments == 0) return sgg::ok();
  SGG_CHECK(workspace == nullptr || sgg::aligned16(workspace), SGG_ERR_UNSUPPORTED,
            "workspace must be 16-byte aligned");
  const int64_t part_avail = workspace_bytes - sgg::kCounterBytes;
  rc = do_shrink(x, ldx, A, h, ldh, s, in_dim, num_loras, num_slices, R, seg_indptr, seg_slots,
                 num_segments, permutation, lora_ranks, chunk_size,
                 static_cast<int32_t*>(workspace),
                 workspace && part_avail > 0 ? static_cast<char*>(workspace) + sgg::kCounterBytes
                                             : nullptr,
                 part_avail, static_cast<hipStream_t>(stream));
  return rc ? rc : sgg::ok();
}

extern "C" int lora_expand(const void* h, int64_t ldh, const void* B, int64_t N,
                           void* base_output, int64_t ldo, int64_t s, int32_t num_loras,
                           int32_t R, const int32_t* slice_offsets, int32_t num_slices,
                           int32_t max_slice_size, const int32_t* seg_indptr,
                           const int32_t* seg_slots, int32_t num_segments,
                           const int32_t* permutation, const int32_t* lora_ranks,
                           const float* scalings, int32_t chunk_size, void* stream) {
  int rc = check_plan(s, num_segments, seg_indptr, seg_slots, permutation, lora_ranks, num_loras,
                      chunk_size);
  if (rc) return rc;
  rc = check_expand(h, ldh, B, N, base_output, ldo, R, slice_offsets, num_slices, max_slice_size,
                    scalings, s);
  if (rc) return rc;
  if (s == 0 || num_segments == 0 || slice_offsets[num_slices] == 0) return sgg::ok();
  rc = do_expand(h, ldh, B, N, base_output, ldo, s, num_loras, R, slice_offsets, num_slices,
                 seg_indptr, seg_slots, num_segments, permutation, lora_ranks, scalings,
                 nullptr, 0, static_cast<hipStream_t>(stream));
  return rc ? rc : sgg::ok();
}

namespace {

// The stacked shrink + expand of lora_qkv, over s output rows; output row r
// reads x row r / xdiv (x has x_rows rows): 1 for lora_qkv, top_k for the
// MoE LoRA add, whose output rows are a token's top-k copies.
int stacked_call(const void* x, int64_t ldx, int64_t x_rows, int32_t xdiv, const void* A,
                 const void* B, int64_t N, void* base_output, int64_t ldo, int64_t s,
                 int64_t in_dim, int32_t num_loras, int32_t R, const int32_t* slice_offsets,
                 int32_t num_slices, int32_t max_slice_size, const int32_t* seg_indptr,
                 const int32_t* seg_slots, int32_t num_segments, const int32_t* permutation,
                 const int32_t* lora_ranks, const float* scalings, int32_t chunk_size,
                 void* workspace, int64_t workspace_bytes, void* stream) {
  int rc = check_plan(s, num_segments, seg_indptr, seg_slots, permutation, lora_ranks, num_loras,
                      chunk_size);
  if (rc) return rc;
  const int64_t hbytes = sgg::round_up(s * num_slices * R * 2, 256);
  SGG_CHECK(workspace != nullptr || s == 0, SGG_ERR_INVALID, "workspace is NULL");
  SGG_CHECK(workspace == nullptr || sgg::aligned16(workspace), SGG_ERR_UNSUPPORTED,
            "workspace must be 16-byte aligned");
  const void* hcheck = workspace ? static_cast<const void*>(static_cast<char*>(workspace) +
                                                            sgg::kCounterBytes)
                                 : x;
  rc = check_shrink(x, ldx, A, hcheck, static_cast<int64_t>(num_slices) * R, s, in_dim,
                    num_loras, num_slices, R);
  if (rc) return rc;
  rc = check_expand(hcheck, static_cast<int64_t>(num_slices) * R, B, N, base_output, ldo, R,
                    slice_offsets, num_slices, max_slice_size, scalings, s);
  if (rc) return rc;
  if (s == 0 || num_segments == 0) return sgg::ok();
  const int64_t need = lora_qkv_workspace_bytes(s, in_dim, num_slices, R, num_segments, chunk_size);
  SGG_CHECK(workspace_bytes >= need, SGG_ERR_CAPACITY,
            "qkv workspace of %" PRId64 " bytes needed, %" PRId64 " given", need, workspace_bytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Workspace: [split-K counters][h, s x c*R bf16][split-K partials].  With
  // K split, the expand sums the shrink's partials itself (h is not written).
  char* ws = static_cast<char*>(workspace);
  int32_t* counters = reinterpret_cast<int32_t*>(ws);
  void* h = ws + sgg::kCounterBytes;
  float* part = reinterpret_cast<float*>(ws + sgg::kCounterBytes + hbytes);
  const int64_t CR = static_cast<int64_t>(num_slices) * R;
  const sgg::ShrinkTiling ts = shrink_tiling(
      s, in_dim, num_slices * R, num_segments, chunk_size,
      gemm_addressable(x_rows, ldx, in_dim, CR));
  SGG_CHECK(ts.grid < (int64_t{1} << 31), SGG_ERR_UNSUPPORTED, "shrink grid too large");
  SGG_CHECK(ts.partial_bytes < (int64_t{1} << 32) - 256, SGG_ERR_UNSUPPORTED,
            "split-K partials of %" PRId64 " bytes exceed 32-bit offsets", ts.partial_bytes);
  if (slice_offsets[num_slices] == 0) return sgg::ok();  // no output columns: nothing changes
  const bool split = ts.ksplit > 1;
  sgg::ShrinkParams ps =
      shrink_params(x, ldx, A, h, CR, s, in_dim, num_loras, num_slices, R, seg_indptr,
                    seg_slots, num_segments, permutation, lora_ranks, counters, part, true, ts);
  ps.x_rows = x_rows;
  ps.xdiv = xdiv;
  sgg::ExpandTiling te{};
  const sgg::ExpandParams pe =
      expand_params(h, CR, B, N, base_output, ldo, s, num_loras, R, slice_offsets, num_slices,
                    seg_indptr, seg_slots, num_segments, permutation, lora_ranks, scalings,
                    split ? part : nullptr, ts.ksplit, &te);
  SGG_CHECK(te.grid < (int64_t{1} << 31), SGG_ERR_UNSUPPORTED, "expand grid too large");
  // The one-launch form (fused.hip), when asked for: a small batch whose
  // shrink splits K (e.g. decode) and whose stacked rank rows fit one
  // producer tile (c*R <= 48), if its grid -- producer tiles of its own
  // tiling plus 128-column consumers -- fits on the device at once.  Its K
  // split differs from the two-launch form's, so its bits can differ from
  // it in rounding.  Measured on the decode batch it is slower than the two
  // launches (a longer chain of dependent device-wide memory round trips), so
  // it is off by default.
  if (g_fused_stacked.load(std::memory_order_relaxed) != 0 && split && CR <= 48 && xdiv == 1 &&
      num_segments <= sgg::kFusedMaxSegments) {
    sgg::ExpandTiling tf{};
    sgg::ExpandParams pf =
        expand_params(h, CR, B, N, base_output, ldo, s, num_loras, R, slice_offsets, num_slices,
                      seg_indptr, seg_slots, num_segments, permutation, lora_ranks, scalings,
                      part, 0, &tf, 1, true);
    const sgg::ShrinkTiling tp = tf.ks <= 2
        ? sgg::choose_fused_tiling(s, in_dim, static_cast<int>(CR), num_segments, chunk_size,
                                   tf.grid, tf.ks, -1,
                                   static_cast<int>(g_fused_ksplit.load(std::memory_order_relaxed)))
        : sgg::ShrinkTiling{};
    const int64_t per_seg = static_cast<int64_t>(tp.mblocks) * tp.nblocks * tp.ksplit;
    const int64_t avail = workspace_bytes - sgg::kCounterBytes - hbytes;
    if (tp.grid > 0 && per_seg < 65536 && per_seg + pf.total_tiles < 32768 &&
        tp.grid + tf.grid < (int64_t{1} << 31) && tp.partial_bytes <= avail &&
        tp.partial_bytes < (int64_t{1} << 32) - 256) {
      const sgg::ShrinkParams pp =
          shrink_params(x, ldx, A, h, CR, s, in_dim, num_loras, num_slices, R, seg_indptr,
                        seg_slots, num_segments, permutation, lora_ranks, counters, part, true,
                        tp);
      pf.hsplit = tp.ksplit;
      pf.hpart_bytes = static_cast<uint32_t>(tp.partial_bytes);
      sgg::FusedSync fs{};
      fs.ready = counters + sgg::kFusedReady;
      fs.status = counters + sgg::kFusedStatus;
      fs.producer_blocks = static_cast<int32_t>(tp.grid);
      fs.producers_per_seg = static_cast<int32_t>(per_seg);
      fs.consumers_per_seg = pf.total_tiles;
      fs.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
      fs.trace = reinterpret_cast<uint64_t*>(g_fused_trace.load(std::memory_order_relaxed));
      {
        const int64_t tb = g_fused_trace_blocks.load(std::memory_order_relaxed);
        fs.trace_blocks = fs.trace ? static_cast<int32_t>(tb < (int64_t{1} << 30) ? tb : 0) : 0;
      }
      rc = launch_status(sgg::launch_fused(pp, tp, pf, tf, fs, st), "fused stacked call");
      return rc ? rc : sgg::ok();
    }
  }
  rc = launch_status(sgg::launch_shrink(ps, ts, st), "shrink");
  if (rc) return rc;
  rc = launch_status(sgg::launch_expand(pe, te, st), "expand");
  return rc ? rc : sgg::ok();
}

}  // namespace

extern "C" int lora_qkv(const void* x, int64_t ldx, const void* A, const void* B, int64_t N,
                        void* base_output, int64_t ldo, int64_t s, int64_t in_dim,
                        int32_t num_loras, int32_t R, const int32_t* slice_offsets,
                        int32_t num_slices, int32_t max_slice_size, const int32_t* seg_indptr,
                        const int32_t* seg_slots, int32_t num_segments,
                        const int32_t* permutation, const int32_t* lora_ranks,
                        const float* scalings, int32_t chunk_size, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  return stacked_call(x, ldx, s, 1, A, B, N, base_output, ldo, s, in_dim, num_loras, R,
                      slice_offsets, num_slices, max_slice_size, seg_indptr, seg_slots,
                      num_segments, permutation, lora_ranks, scalings, chunk_size, workspace,
                      workspace_bytes, stream);
}

extern "C" int lora_moe_route(const int32_t* req_seg_indptr, const int32_t* req_weight_indices,
                              int32_t num_reqs, const int32_t* topk_ids, int64_t num_tokens,
                              int32_t top_k, int32_t num_experts, const int32_t* lora_ranks,
                              const float* scalings, int32_t num_loras, int32_t* virtual_slots,
                              int32_t* virtual_ranks, float* virtual_scalings, void* stream) {
  SGG_CHECK(num_reqs >= 0 && num_tokens >= 0, SGG_ERR_INVALID,
            "num_reqs=%d and num_tokens=%" PRId64 " must be non-negative", num_reqs, num_tokens);
  SGG_CHECK(top_k >= 1 && num_experts >= 1 && num_loras >= 1, SGG_ERR_INVALID,
            "top_k=%d, num_experts=%d and num_loras=%d must be positive", top_k, num_experts,
            num_loras);
  SGG_CHECK(num_tokens * top_k <= INT32_MAX, SGG_ERR_UNSUPPORTED,
            "num_tokens * top_k above int32 indexing");
  SGG_CHECK(static_cast<int64_t>(num_loras) * num_experts < INT32_MAX, SGG_ERR_UNSUPPORTED,
            "num_loras * num_experts above int32 indexing");
  SGG_CHECK(req_seg_indptr && lora_ranks && scalings && virtual_ranks && virtual_scalings,
            SGG_ERR_INVALID, "req_seg_indptr, lora_ranks, scalings or a virtual table is NULL");
  SGG_CHECK(req_weight_indices || num_reqs == 0, SGG_ERR_INVALID, "req_weight_indices is NULL");
  SGG_CHECK((topk_ids && virtual_slots) || num_tokens == 0, SGG_ERR_INVALID,
            "topk_ids or virtual_slots is NULL");
  sgg::MoeRouteParams p{};
  p.req_seg_indptr = req_seg_indptr;
  p.req_weight_indices = req_weight_indices;
  p.topk_ids = topk_ids;
  p.ranks = lora_ranks;
  p.scalings = scalings;
  p.slots = virtual_slots;
  p.vranks = virtual_ranks;
  p.vscalings = virtual_scalings;
  p.copies = num_tokens * top_k;
  p.bs = num_reqs;
  p.top_k = top_k;
  p.E = num_experts;
  p.L = num_loras;
  const int rc = launch_status(sgg::launch_moe_route(p, static_cast<hipStream_t>(stream)),
                               "MoE routing");
  return rc ? rc : sgg::ok();
}

extern "C" int lora_moe_plan(const int32_t* req_seg_indptr, const int32_t* req_weight_indices,
                             int32_t num_reqs, const int32_t* topk_ids, int64_t num_tokens,
                             int32_t top_k, int32_t num_experts, const int32_t* lora_ranks,
                             const float* scalings, int32_t num_loras, int32_t max_chunk_size,
                             int32_t seg_capacity, void* device_plan, int64_t buffer_bytes,
                             int32_t* device_info, void* stream) {
  SGG_CHECK(num_reqs >= 0 && num_tokens >= 0, SGG_ERR_INVALID,
            "num_reqs=%d and num_tokens=%" PRId64 " must be non-negative", num_reqs, num_tokens);
  SGG_CHECK(top_k >= 1 && num_experts >= 1 && num_loras >= 1, SGG_ERR_INVALID,
            "top_k=%d, num_experts=%d and num_loras=%d must be positive", top_k, num_experts,
            num_loras);
  const int64_t copies = num_tokens * top_k;
  const int64_t nv = static_cast<int64_t>(num_loras) * num_experts + 1;
  SGG_CHECK(copies <= sgg::kDevicePlanMaxReqs, SGG_ERR_UNSUPPORTED,
            "%" PRId64 " copies above the device planner's %d", copies, sgg::kDevicePlanMaxReqs);
  SGG_CHECK(nv <= sgg::kDevicePlanMaxLoras, SGG_ERR_UNSUPPORTED,
            "num_loras * num_experts + 1 = %" PRId64 " above the device planner's %d", nv,
            sgg::kDevicePlanMaxLoras);
  SGG_CHECK(seg_capacity >= 0, SGG_ERR_INVALID, "seg_capacity=%d is negative", seg_capacity);
  SGG_CHECK(req_seg_indptr && lora_ranks && scalings && device_plan && device_info,
            SGG_ERR_INVALID,
            "req_seg_indptr, lora_ranks, scalings, device_plan or device_info is NULL");
  SGG_CHECK(req_weight_indices || num_reqs == 0, SGG_ERR_INVALID, "req_weight_indices is NULL");
  SGG_CHECK(topk_ids || num_tokens == 0, SGG_ERR_INVALID, "topk_ids is NULL");
  SGG_CHECK((reinterpret_cast<uintptr_t>(device_plan) & 3) == 0, SGG_ERR_INVALID,
            "device_plan must be 4-byte aligned");
  int64_t off[SGG_PLAN_REGIONS];
  lora_plan_layout(copies, seg_capacity, static_cast<int32_t>(copies),
                   static_cast<int32_t>(nv), off);
  SGG_CHECK(buffer_bytes >= off[9] * 4, SGG_ERR_CAPACITY,
            "plan buffer of %" PRId64 " bytes, regions 0-8 need %" PRId64, buffer_bytes,
            off[9] * 4);
  sgg::MoeRouteParams r{};
  r.req_seg_indptr = req_seg_indptr;
  r.req_weight_indices = req_weight_indices;
  r.topk_ids = topk_ids;
  r.ranks = lora_ranks;
  r.scalings = scalings;
  r.copies = copies;
  r.bs = num_reqs;
  r.top_k = top_k;
  r.E = num_experts;
  r.L = num_loras;
  const int rc = launch_status(
      sgg::launch_moe_plan(r, max_chunk_size, seg_capacity, off,
                           static_cast<int32_t*>(device_plan), device_info,
                           static_cast<hipStream_t>(stream)),
      "MoE routing and plan");
  return rc ? rc : sgg::ok();
}

extern "C" int lora_moe_add(const void* x, int64_t ldx, int64_t num_tokens, int32_t top_k,
                            const void* A, const void* B, int64_t N, void* out, int64_t ldo,
                            int64_t in_dim, int32_t num_virtual, int32_t R,
                            const int32_t* seg_indptr, const int32_t* seg_slots,
                            int32_t num_segments, const int32_t* permutation,
                            const int32_t* virtual_ranks, const float* virtual_scalings,
                            int32_t chunk_size, void* workspace, int64_t workspace_bytes,
                            void* stream) {
  SGG_CHECK(num_tokens >= 0 && top_k >= 1, SGG_ERR_INVALID,
            "num_tokens=%" PRId64 " and top_k=%d: need num_tokens >= 0 and top_k >= 1",
            num_tokens, top_k);
  SGG_CHECK(num_tokens * top_k <= INT32_MAX, SGG_ERR_UNSUPPORTED,
            "num_tokens * top_k above int32 indexing");
  SGG_CHECK(N <= INT32_MAX, SGG_ERR_UNSUPPORTED, "N above int32 offsets");
  const int32_t offs[2] = {0, static_cast<int32_t>(N)};
  return stacked_call(x, ldx, num_tokens, top_k, A, B, N, out, ldo, num_tokens * top_k, in_dim,
                      num_virtual, R, offs, 1, static_cast<int32_t>(N), seg_indptr, seg_slots,
                      num_segments, permutation, virtual_ranks, virtual_scalings, chunk_size,
                      workspace, workspace_bytes, stream);
}

extern "C" int64_t lora_set_option(const char* name, int64_t value) {
  if (name == nullptr) return -1;
  if (std::strcmp(name, "fused_stacked") == 0) return g_fused_stacked.exchange(value != 0);
  if (std::strcmp(name, "spin_limit") == 0)
    return g_spin_limit.exchange(value < 0 ? 0 : value);
  if (std::strcmp(name, "fused_ksplit") == 0)
    return g_fused_ksplit.exchange(value < 0 ? 0 : value);
  if (std::strcmp(name, "expand_deal_tiles") == 0)
    return g_expand_deal_tiles.exchange(value != 0);
  if (std::strcmp(name, "shrink_valu") == 0) return g_shrink_valu.exchange(value != 0);
  if (std::strcmp(name, "shrink_pair_tiles") == 0)
    return g_shrink_pair_tiles.exchange(value != 0);
  if (std::strcmp(name, "fused_trace") == 0) return g_fused_trace.exchange(value);
  if (std::strcmp(name, "fused_trace_blocks") == 0)
    return g_fused_trace_blocks.exchange(value < 0 ? 0 : value);
  return -1;
}

// ------------------------------------------------------- no-allocation qkv
// lora_qkv for callers that cannot allocate device memory (code under graph
// capture, tight serving loops): the workspace is this file-scope device
// array.  Each device holds its own copy, at its own address, for the life
// of the process; host code uses that address (looked up once per device with
// the device current), never the array's name, which on the host is only a
// stand-in.  The array is zero when the module loads, and every lora_qkv call
// leaves its counter region at zero again, which is all a call needs to find
// at its start; h and the partials are written before they are read.  Calls
// on one device share the array: calls that overlap in time race.

namespace {

static __device__ __align__(256) char scratch[SGG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device); nullptr with the error recorded on failure.
void* scratch_for_current_device(int* rc) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = fail(SGG_ERR_HIP, "no current device for the scratch array (%s)",
               e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *rc = fail(SGG_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                 hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int lora_qkv_noalloc(const void* x, int64_t ldx, const void* A, const void* B,
                                int64_t N, void* base_output, int64_t ldo, int64_t s,
                                int64_t in_dim, int32_t num_loras, int32_t R,
                                const int32_t* slice_offsets, int32_t num_slices,
                                int32_t max_slice_size, const int32_t* seg_indptr,
                                const int32_t* seg_slots, int32_t num_segments,
                                const int32_t* permutation, const int32_t* lora_ranks,
                                const float* scalings, int32_t chunk_size, void* stream) {
  const int64_t need =
      lora_qkv_workspace_bytes(s, in_dim, num_slices, R, num_segments, chunk_size);
  SGG_CHECK(need <= SGG_NOALLOC_SCRATCH_BYTES, SGG_ERR_CAPACITY,
            "lora_qkv_noalloc needs %" PRId64 " bytes of scratch, its maximum is %lld; "
            "call lora_qkv with a workspace instead",
            need, static_cast<long long>(SGG_NOALLOC_SCRATCH_BYTES));
  int rc = SGG_OK;
  void* ws = scratch_for_current_device(&rc);
  if (ws == nullptr) return rc;
  return lora_qkv(x, ldx, A, B, N, base_output, ldo, s, in_dim, num_loras, R, slice_offsets,
                  num_slices, max_slice_size, seg_indptr, seg_slots, num_segments, permutation,
                  lora_ranks, scalings, chunk_size, ws, SGG_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int lora_a_embedding(const int64_t* input_ids, const void* A_emb, int64_t V, void* out,
                                int64_t ldo, int64_t s, int32_t num_loras, int32_t R,
                                int64_t vocab_size, const int32_t* seg_indptr,
                                const int32_t* seg_slots, int32_t num_segments,
                                const int32_t* permutation, const int32_t* lora_ranks,
                                int32_t has_extra_embeddings, void* stream) {
  SGG_CHECK(!has_extra_embeddings, SGG_ERR_UNSUPPORTED,
            "extra (added-vocabulary) embeddings are not supported by the chunked backend");
  int rc = check_plan(s, num_segments, seg_indptr, seg_slots, permutation, lora_ranks, num_loras,
                      1);
  if (rc) return rc;
  SGG_CHECK(A_emb && ((input_ids && out) || s == 0), SGG_ERR_INVALID,
            "input_ids, A_emb or out is NULL");
  SGG_CHECK(R > 0, SGG_ERR_INVALID, "R=%d must be positive", R);
  SGG_CHECK(vocab_size >= 0 && vocab_size <= V, SGG_ERR_INVALID,
            "vocab_size=%" PRId64 " outside [0, V=%" PRId64 "]", vocab_size, V);
  SGG_CHECK(ldo >= R, SGG_ERR_INVALID, "ldo=%" PRId64 " < R=%d", ldo, R);
  SGG_CHECK((reinterpret_cast<uintptr_t>(out) & 1u) == 0 &&
                (reinterpret_cast<uintptr_t>(A_emb) & 1u) == 0 &&
                (reinterpret_cast<uintptr_t>(input_ids) & 7u) == 0,
            SGG_ERR_UNSUPPORTED, "misaligned pointer");
  if (s == 0 || num_segments == 0) return sgg::ok();
  sgg::EmbeddingParams p{};
  p.ids = input_ids;
  p.A = static_cast<const uint16_t*>(A_emb);
  p.out = static_cast<uint16_t*>(out);
  p.seg_indptr = seg_indptr;
  p.seg_slots = seg_slots;
  p.perm = permutation;
  p.ranks = lora_ranks;
  p.V = V;
  p.vocab = vocab_size;
  p.ldo = ldo;
  p.s = s;
  p.L = num_loras;
  p.R = R;
  p.num_segments = num_segments;
  // Plans of more segments than the position-major form takes (see
  // launch_embedding) run segment-major, with parts per segment: about 64
  // (token, j) pairs per workgroup.  Every pair
  // is its own cache line (A_emb columns are V apart) and one CU keeps only
  // so many line requests in flight, so the gather is spread over many CUs.
  // Measured on the decode batch (256 tokens, 8 segments, R = 16): 4.4 us
  // with about 1024 pairs per workgroup, 3.0 us with 64 or 128; the
  // full-layer batch (4288 tokens) 9.1 -> 8.9 us.
  const int64_t avg = (s + num_segments - 1) / num_segments;
  int64_t parts = (avg * R + 63) / 64;
  p.parts = static_cast<int32_t>(parts < 1 ? 1 : (parts > 64 ? 64 : parts));
  rc = launch_status(sgg::launch_embedding(p, static_cast<hipStream_t>(stream)), "embedding");
  return rc ? rc : sgg::ok();
}

// ------------------------------------------------------------- plan upload

extern "C" int64_t lora_plan_layout(int64_t token_capacity, int32_t seg_capacity,
                                    int32_t req_capacity, int32_t max_loras, int64_t* offsets) {
  if (token_capacity < 0 || seg_capacity < 0 || req_capacity < 0 || max_loras < 0) return -1;
  const int64_t sizes[SGG_PLAN_REGIONS] = {token_capacity, seg_capacity + 1, seg_capacity,
                                           req_capacity + 1, req_capacity, max_loras, max_loras,
                                           seg_capacity + 1, seg_capacity, token_capacity};
  int64_t pos = 0;
  for (int i = 0; i < SGG_PLAN_REGIONS; ++i) {
    if (offsets) offsets[i] = pos;
    pos += sgg::round_up(sizes[i], 64);
  }
  return pos;
}

namespace {

// The LoRA-A embedding lookup that lora_plan_upload_embedding runs over the
// batch it uploads (arguments as lora_a_embedding's, already checked).
struct EmbedRequest {
  const int64_t* ids;
  const void* A;
  int64_t V;
  void* out;
  int64_t ldo;
  int32_t R;
  int64_t vocab;
};

// Plan into the staging buffer (`lm_head`: the pruned lm_head plan, else the
// chunked plan), add the tables and the work segments, then one transfer
// (and, given `emb`, the embedding lookup over the uploaded plan).
int plan_upload(bool lm_head, const int32_t* seq_lens, const int32_t* req_slots,
                int32_t num_reqs, const int32_t* lora_ranks, const float* scalings,
                int32_t max_loras, int32_t is_decode, int32_t max_chunk_size,
                int32_t chunk_size_override, int64_t token_capacity, int32_t seg_capacity,
                int32_t req_capacity, void* host_staging, void* device_plan,
                int64_t buffer_bytes, int32_t* out_info, int32_t* done_flag,
                int32_t done_value, void* stream, const EmbedRequest* emb = nullptr) {

  int64_t off[SGG_PLAN_REGIONS];
  const int64_t total = lora_plan_layout(token_capacity, seg_capacity, req_capacity, max_loras, off);
  SGG_CHECK(total >= 0, SGG_ERR_INVALID, "negative capacity");
  SGG_CHECK(host_staging && device_plan && out_info, SGG_ERR_INVALID,
            "host_staging, device_plan or out_info is NULL");
  SGG_CHECK(lora_ranks && scalings, SGG_ERR_INVALID, "lora_ranks or scalings is NULL");
  SGG_CHECK(((reinterpret_cast<uintptr_t>(host_staging) | reinterpret_cast<uintptr_t>(device_plan)) &
             7) == 0,
            SGG_ERR_INVALID, "host_staging and device_plan must be 8-byte aligned");
  int32_t* done_dev = nullptr;
  if (done_flag != nullptr) {
    void* m = nullptr;
    const hipError_t me = hipHostGetDevicePointer(&m, done_flag, 0);
    if (me != hipSuccess || m == nullptr) {
      (void)hipGetLastError();
      return fail(SGG_ERR_INVALID, "done_flag is not pinned host memory mapped for the device");
    }
    done_dev = static_cast<int32_t*>(m);
  }
  SGG_CHECK(buffer_bytes >= total * 4, SGG_ERR_CAPACITY,
            "plan buffer of %" PRId64 " bytes, layout needs %" PRId64, buffer_bytes, total * 4);
  SGG_CHECK(num_reqs <= req_capacity, SGG_ERR_CAPACITY, "%d requests > capacity %d", num_reqs,
            req_capacity);
  int32_t* h = static_cast<int32_t*>(host_staging);
  int32_t n_seg = 0, chunk = 0;
  int64_t n_tok = 0;
  int rc;
  if (lm_head) {
    rc = lora_plan_lm_head(seq_lens, req_slots, num_reqs, max_loras, max_chunk_size,
                           chunk_size_override, h + off[0], token_capacity, h + off[1],
                           h + off[2], seg_capacity, &n_seg, &chunk, &n_tok);
    if (rc == 0) {  // request boundaries over the pruned tokens
      int64_t acc = 0;
      h[off[3]] = 0;
      for (int32_t r = 0; r < num_reqs; ++r) {
        acc += seq_lens[r];
        h[off[3] + r + 1] = static_cast<int32_t>(acc);
      }
    }
  } else {
    rc = lora_plan_segments(seq_lens, req_slots, num_reqs, max_loras, is_decode, max_chunk_size,
                            chunk_size_override, h + off[0], token_capacity, h + off[1],
                            h + off[2], seg_capacity, h + off[3], &n_seg, &chunk, &n_tok);
  }
  if (rc) return rc;
  for (int32_t r = 0; r < num_reqs; ++r) h[off[4] + r] = req_slots[r];
  for (int32_t a = 0; a < max_loras; ++a) h[off[5] + a] = lora_ranks[a];
  std::memcpy(h + off[6], scalings, sizeof(float) * static_cast<size_t>(max_loras));
  int32_t longest = 0;
  for (int32_t i = 0; i < n_seg; ++i) {
    const int32_t len = h[off[1] + i + 1] - h[off[1] + i];
    longest = len > longest ? len : longest;
  }
  // Work segments: merge consecutive segments of one slot up to `cap` tokens.
  // For the lm_head plan they come from the pruned tokens sorted by slot (a
  // stable sort, whose permutation goes to region 9): its identity order
  // leaves runs of about one token wherever adapters interleave, and every
  // run would re-read its adapter's B tile across the whole vocabulary.
  const int32_t* sind = h + off[1];
  const int32_t* sslot = h + off[2];
  int32_t n_src = n_seg;
  if (lm_head) {
    thread_local std::vector<int32_t> sorted;
    sorted.resize(2 * static_cast<size_t>(seg_capacity) + static_cast<size_t>(num_reqs) + 2);
    int32_t* tind = sorted.data();
    int32_t* tslot = tind + seg_capacity + 1;
    int32_t* treq = tslot + seg_capacity;
    int32_t ts = 0, tchunk = 0;
    int64_t ttok = 0;
    rc = lora_plan_segments(seq_lens, req_slots, num_reqs, max_loras, 0, max_chunk_size,
                            chunk_size_override, h + off[9], token_capacity, tind, tslot,
                            seg_capacity, treq, &ts, &tchunk, &ttok);
    if (rc) return rc;
    sind = tind;
    sslot = tslot;
    n_src = ts;
  }
  int32_t* wind = h + off[7];
  int32_t* wslot = h + off[8];
  const int32_t cap = chunk > SGG_WORK_SEGMENT_TOKENS ? chunk : SGG_WORK_SEGMENT_TOKENS;
  int32_t n_work = 0, longest_work = 0;
  wind[0] = 0;
  for (int32_t i = 0; i < n_src;) {
    int32_t j = i + 1;
    while (j < n_src && sslot[j] == sslot[i] && sind[j + 1] - sind[i] <= cap) ++j;
    wslot[n_work] = sslot[i];
    wind[n_work + 1] = sind[j];
    const int32_t len = sind[j] - sind[i];
    longest_work = len > longest_work ? len : longest_work;
    ++n_work;
    i = j;
  }
  for (int32_t i = n_work; i < seg_capacity; ++i) {
    wslot[i] = 0;
    wind[i + 1] = wind[n_work];
  }
  // One transfer (region 9 only for the lm_head plan): a copy kernel reading
  // the pinned buffer through its device mapping (it also raises the done
  // flag); a runtime copy only if the buffer has no device mapping, followed
  // by an empty copy that raises the flag.  With an embedding request over a
  // decode-shaped batch (token t is request t) of at most
  // kEmbedUploadMaxTokens tokens and kEmbedUploadMaxLoras slots, the copy
  // kernel also does the lookup, from slots and ranks passed as kernel
  // arguments; otherwise the lookup runs after the copy, over the device plan.
  const int64_t n_copy = lm_head ? total : off[9];
  void* src = nullptr;
  hipError_t e = hipHostGetDevicePointer(&src, host_staging, 0);
  const bool mapped = e == hipSuccess && src != nullptr;
  bool decode_shaped = is_decode != 0 || n_tok == num_reqs;
  for (int32_t r = 0; !is_decode && decode_shaped && r < num_reqs; ++r)
    decode_shaped = seq_lens[r] == 1;
  // (the launch indexes its (token, j) pairs and blocks with 32-bit ints)
  const bool fused_embed = emb != nullptr && mapped && !lm_head && decode_shaped && n_tok > 0 &&
                           n_tok <= sgg::kEmbedUploadMaxTokens &&
                           max_loras <= sgg::kEmbedUploadMaxLoras &&
                           n_tok * emb->R <= int64_t{INT32_MAX} - 256;
  if (fused_embed) {
    sgg::EmbedUploadParams ep;
    ep.src = static_cast<const int32_t*>(src);
    ep.dst = static_cast<int32_t*>(device_plan);
    ep.done = done_dev;
    ep.ids = emb->ids;
    ep.A = static_cast<const uint16_t*>(emb->A);
    ep.out = static_cast<uint16_t*>(emb->out);
    ep.n = n_copy;
    ep.V = emb->V;
    ep.vocab = emb->vocab;
    ep.ldo = emb->ldo;
    ep.done_value = done_value;
    ep.s = static_cast<int32_t>(n_tok);
    ep.R = emb->R;
    ep.pad_ = 0;
    for (int32_t a = 0; a < sgg::kEmbedUploadMaxLoras; ++a) {
      const int32_t rho = a < max_loras ? lora_ranks[a] : 0;
      ep.rank[a] = rho < 0 ? 0 : (rho > emb->R ? emb->R : rho);
    }
    // the planner has checked every slot against max_loras (<= 64)
    for (int32_t t = 0; t < ep.s; ++t) ep.slot[t] = static_cast<uint8_t>(req_slots[t]);
    e = sgg::launch_plan_copy_embedding(ep, static_cast<hipStream_t>(stream));
  } else if (mapped) {
    e = sgg::launch_plan_copy(static_cast<const int32_t*>(src), static_cast<int32_t*>(device_plan),
                              n_copy, done_dev, done_value, static_cast<hipStream_t>(stream));
  } else {
    (void)hipGetLastError();  // clear the failed lookup
    e = hipMemcpyAsync(device_plan, host_staging, static_cast<size_t>(n_copy) * 4,
                       hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (e == hipSuccess && done_dev != nullptr)
      e = sgg::launch_plan_copy(nullptr, nullptr, 0, done_dev, done_value,
                                static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess)
    return fail(SGG_ERR_HIP, "plan upload failed: %s", hipGetErrorString(e));
  out_info[0] = n_seg;
  out_info[1] = chunk;
  out_info[2] = longest;
  out_info[3] = static_cast<int32_t>(n_tok);
  out_info[4] = n_work;
  out_info[5] = longest_work;
  if (emb != nullptr && !fused_embed && n_tok > 0) {
    const int32_t* d = static_cast<const int32_t*>(device_plan);
    return lora_a_embedding(emb->ids, emb->A, emb->V, emb->out, emb->ldo, n_tok, max_loras,
                            emb->R, emb->vocab, d + off[1], d + off[2], n_seg, d + off[0],
                            d + off[5], 0, stream);
  }
  return sgg::ok();
}

}  // namespace

extern "C" int lora_plan_upload(const int32_t* seq_lens, const int32_t* req_slots,
                                int32_t num_reqs, const int32_t* lora_ranks,
                                const float* scalings, int32_t max_loras, int32_t is_decode,
                                int32_t max_chunk_size, int32_t chunk_size_override,
                                int64_t token_capacity, int32_t seg_capacity,
                                int32_t req_capacity, void* host_staging, void* device_plan,
                                int64_t buffer_bytes, int32_t* out_info, int32_t* done_flag,
                                int32_t done_value, void* stream) {
  return plan_upload(false, seq_lens, req_slots, num_reqs, lora_ranks, scalings, max_loras,
                     is_decode, max_chunk_size, chunk_size_override, token_capacity,
                     seg_capacity, req_capacity, host_staging, device_plan, buffer_bytes,
                     out_info, done_flag, done_value, stream);
}

extern "C" int lora_plan_upload_embedding(
    const int32_t* seq_lens, const int32_t* req_slots, int32_t num_reqs,
    const int32_t* lora_ranks, const float* scalings, int32_t max_loras, int32_t is_decode,
    int32_t max_chunk_size, int32_t chunk_size_override, int64_t token_capacity,
    int32_t seg_capacity, int32_t req_capacity, void* host_staging, void* device_plan,
    int64_t buffer_bytes, int32_t* out_info, int32_t* done_flag, int32_t done_value,
    const int64_t* input_ids, const void* A_emb, int64_t V, void* out, int64_t ldo, int32_t R,
    int64_t vocab_size, void* stream) {
  // the lookup's arguments are checked before anything is planned or enqueued
  SGG_CHECK(A_emb && ((input_ids && out) || num_reqs == 0), SGG_ERR_INVALID,
            "input_ids, A_emb or out is NULL");
  SGG_CHECK(R > 0, SGG_ERR_INVALID, "R=%d must be positive", R);
  SGG_CHECK(vocab_size >= 0 && vocab_size <= V, SGG_ERR_INVALID,
            "vocab_size=%" PRId64 " outside [0, V=%" PRId64 "]", vocab_size, V);
  SGG_CHECK(ldo >= R, SGG_ERR_INVALID, "ldo=%" PRId64 " < R=%d", ldo, R);
  SGG_CHECK((reinterpret_cast<uintptr_t>(out) & 1u) == 0 &&
                (reinterpret_cast<uintptr_t>(A_emb) & 1u) == 0 &&
                (reinterpret_cast<uintptr_t>(input_ids) & 7u) == 0,
            SGG_ERR_UNSUPPORTED, "misaligned pointer");
  const EmbedRequest emb{input_ids, A_emb, V, out, ldo, R, vocab_size};
  return plan_upload(false, seq_lens, req_slots, num_reqs, lora_ranks, scalings, max_loras,
                     is_decode, max_chunk_size, chunk_size_override, token_capacity,
                     seg_capacity, req_capacity, host_staging, device_plan, buffer_bytes,
                     out_info, done_flag, done_value, stream, &emb);
}

extern "C" int lora_plan_device(const int32_t* seq_lens, const int32_t* req_slots,
                                int32_t num_reqs, const int32_t* lora_ranks,
                                const float* scalings, int32_t max_loras, int32_t is_decode,
                                int32_t max_chunk_size, int32_t chunk_size_override,
                                int64_t token_capacity, int32_t seg_capacity,
                                int32_t req_capacity, void* device_plan, int64_t buffer_bytes,
                                int32_t* device_info, void* stream) {
  int64_t off[SGG_PLAN_REGIONS];
  const int64_t total = lora_plan_layout(token_capacity, seg_capacity, req_capacity, max_loras, off);
  SGG_CHECK(total >= 0, SGG_ERR_INVALID, "negative capacity");
  SGG_CHECK(max_loras >= 1 && max_loras <= sgg::kDevicePlanMaxLoras, SGG_ERR_UNSUPPORTED,
            "max_loras=%d outside [1, %d] for the device planner", max_loras,
            sgg::kDevicePlanMaxLoras);
  SGG_CHECK(num_reqs >= 0 && num_reqs <= sgg::kDevicePlanMaxReqs, SGG_ERR_UNSUPPORTED,
            "num_reqs=%d outside [0, %d] for the device planner", num_reqs,
            sgg::kDevicePlanMaxReqs);
  SGG_CHECK(num_reqs <= req_capacity, SGG_ERR_CAPACITY, "%d requests > capacity %d", num_reqs,
            req_capacity);
  SGG_CHECK(token_capacity <= INT32_MAX, SGG_ERR_INVALID, "token_capacity above int32 indexing");
  SGG_CHECK(num_reqs == 0 || req_slots != nullptr, SGG_ERR_INVALID, "req_slots is NULL");
  SGG_CHECK(is_decode || num_reqs == 0 || seq_lens != nullptr, SGG_ERR_INVALID,
            "seq_lens is NULL in extend mode");
  SGG_CHECK(lora_ranks && scalings && device_plan && device_info, SGG_ERR_INVALID,
            "lora_ranks, scalings, device_plan or device_info is NULL");
  SGG_CHECK(chunk_size_override >= 0, SGG_ERR_INVALID, "chunk_size_override=%d is negative",
            chunk_size_override);
  SGG_CHECK((reinterpret_cast<uintptr_t>(device_plan) & 3) == 0, SGG_ERR_INVALID,
            "device_plan must be 4-byte aligned");
  SGG_CHECK(buffer_bytes >= off[9] * 4, SGG_ERR_CAPACITY,
            "plan buffer of %" PRId64 " bytes, regions 0-8 need %" PRId64, buffer_bytes,
            off[9] * 4);
  const hipError_t e = sgg::launch_plan_device(
      is_decode ? nullptr : seq_lens, req_slots, num_reqs, lora_ranks, scalings, max_loras,
      is_decode, max_chunk_size, chunk_size_override, token_capacity, seg_capacity, off,
      static_cast<int32_t*>(device_plan), device_info, static_cast<hipStream_t>(stream));
  return launch_status(e, "plan_device");
}

extern "C" int lora_plan_lm_head_upload(const int32_t* pruned_lens, const int32_t* req_slots,
                                        int32_t num_reqs, const int32_t* lora_ranks,
                                        const float* scalings, int32_t max_loras,
                                        int32_t max_chunk_size, int32_t chunk_size_override,
                                        int64_t token_capacity, int32_t seg_capacity,
                                        int32_t req_capacity, void* host_staging,
                                        void* device_plan, int64_t buffer_bytes,
                                        int32_t* out_info, int32_t* done_flag,
                                        int32_t done_value, void* stream) {
  SGG_CHECK(num_reqs == 0 || pruned_lens != nullptr, SGG_ERR_INVALID, "pruned_lens is NULL");
  return plan_upload(true, pruned_lens, req_slots, num_reqs, lora_ranks, scalings, max_loras, 0,
                     max_chunk_size, chunk_size_override, token_capacity, seg_capacity,
                     req_capacity, host_staging, device_plan, buffer_bytes, out_info, done_flag,
                     done_value, stream);
}
