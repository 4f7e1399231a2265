// Kernel parameter blocks and host launchers (internal to libsgg_lora).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sgg {

constexpr int kMaxSlices = 8;
constexpr int kXcdCount = 8;  // MI355X: XCDs, each with its own L2 (blocks dealt b % 8)
// Counters sit in a fixed region at the start of every workspace, so a
// counter location never holds anything but a counter (each call leaves its
// counters at zero) whatever the shapes of earlier calls.  Words [0, 8192):
// split-K arrival counters; [8192, 16383): the fused stacked call's
// per-segment hand-off words; word 16383: its give-up status (sticky; byte
// offset SGG_WORKSPACE_STATUS_OFFSET).
constexpr int64_t kCounterBytes = 65536;
constexpr int kCounterCap = 8192;
constexpr int kFusedReady = 8192;
constexpr int kFusedStatus = 16383;
constexpr int kFusedMaxSegments = kFusedStatus - kFusedReady;

// LoRA-A shrink over the segments of a plan.
struct ShrinkParams {
  const uint16_t* x;          // (s, K) bf16, row stride ldx
  const uint16_t* A;          // (L, CR, K) bf16
  uint16_t* h;                // (s, CR) bf16, row stride ldh
  float* partial;             // [ksplit][s][CR] f32 (ksplit > 1)
  int32_t* counters;          // arrival counters per (row block, column block)
  const int32_t* seg_indptr;  // [num_segments + 1]
  const int32_t* seg_slots;   // [num_segments]
  const int32_t* perm;        // [s]
  const int32_t* ranks;       // [L]
  int64_t ldx, ldh, s, K, kps;
  int32_t L, R, CR, num_segments;
  int32_t mblocks;            // row blocks per segment covered by the grid
  int32_t nblocks;            // column blocks over CR
  int32_t ksplit;             // K ranges (one workgroup each)
  int32_t counter_cap;        // entries in `counters`
  int32_t partials_only;      // ksplit > 1: leave the partials for the expand, write no h
  uint32_t partial_bytes;     // size of `partial` (below 2^32)
  // Row of x read for output row r: r / xdiv (1 normally; the MoE LoRA add
  // has top_k output rows per token, x_rows = s / top_k rows of x).
  int64_t x_rows;
  int32_t xdiv;
};

// LoRA-B expand (scale, add into base) over the segments of a plan.
struct ExpandParams {
  const uint16_t* h;          // (s, c*R) bf16, row stride ldh
  const uint16_t* B;          // (L, N, R) bf16
  uint16_t* out;              // (s, >= offs[c]) bf16, row stride ldo
  const int32_t* seg_indptr;
  const int32_t* seg_slots;
  const int32_t* perm;
  const int32_t* ranks;
  const float* scalings;
  // Optional: h as the shrink's f32 split-K partials [hsplit][s][ldp], rows
  // in sorted (plan) order; summed in split order and rounded to bf16 while
  // staging, exactly as the shrink's own reduction would.  Null: read h.
  const float* hpart;
  int64_t ldp;
  int32_t hsplit;
  uint32_t hpart_bytes;       // size of the partials (below 2^32)
  int64_t ldh, ldo, s, N;
  int32_t L, R, c, num_segments;
  int32_t vec8;               // 16-byte base access is aligned for every group of 8 columns
  int32_t offs[kMaxSlices + 1];
  int32_t tile_start[kMaxSlices + 1];  // first column tile of each slice
  int32_t total_tiles;
  int32_t tiles_per_xcd;      // > 0: column tiles dealt to the XCDs (expand_item_of)
};
// Cross-workgroup hand-off of the fused stacked call (fused.hip): producer
// blocks [0, producer_blocks) run the split-K shrink tiles and count
// themselves in bits 0-15 of their segment's word ready[seg] once their
// partials are published; consumer blocks run the expand tiles and wait for
// that count to reach producers_per_seg before staging h.  Every block of a
// segment also counts itself in bits 16-30; the last of the
// producers_per_seg + consumers_per_seg resets the word to zero.  A wait
// gives up after spin_limit polls: the consumer then computes its segment's
// partials itself (the same bits) and sets bit 0 of *status.
struct FusedSync {
  int32_t* ready;
  int32_t* status;
  int32_t producer_blocks;
  int32_t producers_per_seg;
  int32_t consumers_per_seg;
  int64_t spin_limit;
  // Optional block timeline (null: off): block b < trace_blocks writes four
  // 64-bit words at trace + 4b -- start, wait done (producers: work done),
  // end, in ticks of the 100 MHz real-time counter, and its role (0 producer,
  // 1 consumer, 2 consumer that gave up waiting).
  uint64_t* trace;
  int32_t trace_blocks;
};

// Grid of a segment_round_robin launch: whole rounds of 8 segments.
inline int64_t grid_for(int num_segments, int64_t per_segment) {
  return static_cast<int64_t>((num_segments + 7) / 8) * 8 * per_segment;
}

// LoRA-A embedding lookup over the segments of a plan.
struct EmbeddingParams {
  const int64_t* ids;
  const uint16_t* A;          // (L, R, V) bf16
  uint16_t* out;              // (s, R) bf16, row stride ldo
  const int32_t* seg_indptr;
  const int32_t* seg_slots;
  const int32_t* perm;
  const int32_t* ranks;
  int64_t V, vocab, ldo, s;
  int32_t L, R, num_segments, parts;
};

// Tile choice for the shrink (also sizes its workspace).
struct ShrinkTiling {
  int gemm;          // 1: shrink_gemm_kernel with bm x bn tiles; 0: split-K shrink_kernel
  int bm, bn;        // gemm tile (tokens x stacked rank rows); bm = 256: segment pairs, K split
  int mf, nf;        // split-K kernel: row / column fragments of 16
  int mblocks, nblocks, ksplit;
  int64_t kps;
  int64_t partial_bytes;     // f32 partial tiles (0 unless ksplit > 1)
  int64_t grid;
  int valu;          // split-K kernel: tiles of at most 4 tokens on the VALU (mf 1, nf <= 3)
};
// gemm_ok: the GEMM tiles may be chosen (their buffer loads address x and
// each slot's A block with 32-bit byte offsets).  pair_ok: the GEMM tiles
// over segment pairs with K split (bm = 256) may be chosen; they need a
// split-K workspace (partial_bytes) where the other GEMM tiles need none.
ShrinkTiling choose_shrink_tiling(int64_t s, int64_t K, int CR, int num_segments, int chunk,
                                  bool gemm_ok = true, bool pair_ok = false);
// Re-tile a split-K kernel tiling to 16-token tiles whose short tiles (at
// most 4 tokens) compute on the VALU; unchanged where that kernel form does
// not apply (GEMM tiles, more than 48 rank rows per tile, too many arrival
// counters).
void use_valu_tiles(ShrinkTiling* t, int64_t s, int num_segments, int chunk);

struct ExpandTiling {
  int pairs, ks;     // 32-column fragment pairs per wave, 32-deep rank steps
  int64_t grid;
};

// MoE routing: per top-k copy of every token, its virtual expert (adapter x
// expert) from the per-request routing fields; and the virtual rank /
// scaling tables (L*E entries plus one of rank 0 for copies without a valid
// adapter or expert).
struct MoeRouteParams {
  const int32_t* req_seg_indptr;      // [bs + 1]
  const int32_t* req_weight_indices;  // [bs]
  const int32_t* topk_ids;            // [tokens][top_k]
  const int32_t* ranks;               // [L]
  const float* scalings;              // [L]
  int32_t* slots;                     // [tokens * top_k] out
  int32_t* vranks;                    // [L * E + 1] out
  float* vscalings;                   // [L * E + 1] out
  int64_t copies;                     // tokens * top_k
  int32_t bs, top_k, E, L;
};
hipError_t launch_moe_route(const MoeRouteParams& p, hipStream_t stream);

hipError_t launch_shrink(const ShrinkParams& p, const ShrinkTiling& t, hipStream_t stream);
hipError_t launch_shrink_gemm(const ShrinkParams& p, int bm, int bn, int64_t grid,
                              hipStream_t stream);
hipError_t launch_expand(const ExpandParams& p, const ExpandTiling& t, hipStream_t stream);
hipError_t launch_embedding(const EmbeddingParams& p, hipStream_t stream);

// The stacked shrink + expand in one launch (fused.hip): producer tiles of
// 16*mf tokens x 16*nf rank rows (mf <= 2, nf <= 3; partials only), consumer
// tiles of 128 columns (pairs = 1, ks <= 2), at most kFusedMaxSegments
// segments.  fused_resident_blocks() is how many blocks of that launch the
// device keeps resident at once (0 if unknown or no such instance); the host
// takes the fused launch only when the whole grid fits.
int64_t fused_resident_blocks(int mf, int nf, int ks);
// Producer tiling of the fused launch for a batch whose shrink splits K:
// 16*mf tokens x all c*R rank rows per tile, and the largest K split (at
// most kFusedMaxSplit ranges of at least 256, or `force_ksplit` if > 0)
// whose grid, with `consumers` expand blocks, fits `resident` blocks
// (resident < 0: query fused_resident_blocks).  grid == 0: no fused launch.
constexpr int kFusedMaxSplit = 16;
ShrinkTiling choose_fused_tiling(int64_t s, int64_t K, int CR, int num_segments, int chunk,
                                 int64_t consumers, int ks, int64_t resident, int force_ksplit);
hipError_t launch_fused(const ShrinkParams& ps, const ShrinkTiling& ts, const ExpandParams& pe,
                        const ExpandTiling& te, const FusedSync& fs, hipStream_t stream);

// The batch plan on the GPU (plan_device.hip): one workgroup; up to
// kDevicePlanMaxReqs requests and kDevicePlanMaxLoras slots.
constexpr int kDevicePlanMaxLoras = 1024;  // SGG_DEVICE_PLAN_MAX_LORAS
constexpr int kDevicePlanMaxReqs = 4096;   // SGG_DEVICE_PLAN_MAX_REQS
hipError_t launch_plan_device(const int32_t* seq_lens, const int32_t* req_slots, int32_t bs,
                              const int32_t* ranks, const float* scalings, int32_t L,
                              int32_t is_decode, int32_t max_chunk, int32_t chunk_override,
                              int64_t token_capacity, int32_t seg_capacity, const int64_t* off,
                              int32_t* plan, int32_t* info, hipStream_t stream);
// The MoE routing of `r` (its output arrays unused) and the device plan of the
// r.copies one-token copies over the r.L * r.E + 1 virtual slots, in one
// launch of the device planner: regions 0-8 as launch_plan_device over the
// routed slots, the virtual rank / scaling tables in regions 5 and 6.
hipError_t launch_moe_plan(const MoeRouteParams& r, int32_t max_chunk, int32_t seg_capacity,
                           const int64_t* off, int32_t* plan, int32_t* info, hipStream_t stream);

// Copy n int32 from pinned host memory (given by its device-side address) to
// device memory, as a kernel on `stream`; src and dst 8-byte aligned.  When
// done_dev_view is not null (host memory, by its device-side address),
// done_value is written there once the source has been read in full.
hipError_t launch_plan_copy(const int32_t* src_dev_view, int32_t* dst, int64_t n,
                            int32_t* done_dev_view, int32_t done_value, hipStream_t stream);

// The plan copy above and the LoRA-A embedding lookup of a decode-shaped
// batch (token t is request t) in one launch: workgroup 0 copies the plan,
// the others gather the embedding rows.  The per-token slots and the per-slot
// ranks travel in the kernel arguments, so the gather reads neither the plan
// nor the staging buffer: the done flag still means that every read of the
// staging buffer has returned.
constexpr int kEmbedUploadMaxTokens = 3072;
constexpr int kEmbedUploadMaxLoras = 64;
struct EmbedUploadParams {
  const int32_t* src;         // staging buffer, device-side address
  int32_t* dst;               // device plan
  int32_t* done;              // host flag, device-side address (or null)
  const int64_t* ids;
  const uint16_t* A;          // (L, R, V) bf16
  uint16_t* out;              // (s, R) bf16, row stride ldo
  int64_t n, V, vocab, ldo;
  int32_t done_value, s, R, pad_;
  int32_t rank[kEmbedUploadMaxLoras];    // clamped to [0, R]
  uint8_t slot[kEmbedUploadMaxTokens];   // slot of token t
};
hipError_t launch_plan_copy_embedding(const EmbedUploadParams& p, hipStream_t stream);

}  // namespace sgg
