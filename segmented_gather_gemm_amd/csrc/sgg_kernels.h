// Kernel parameter blocks and host launchers (internal to libsgg_lora).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sgg {

constexpr int kMaxSlices = 8;
// Split-K arrival counters sit in a fixed region at the start of every
// workspace, so a counter location never holds anything but a counter (each
// call leaves its counters at zero) whatever the shapes of earlier calls.
constexpr int64_t kCounterBytes = 32768;
constexpr int kCounterCap = static_cast<int>(kCounterBytes / 4);

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
  int64_t ldh, ldo, s, N;
  int32_t L, R, c, num_segments;
  int32_t vec8;               // 16-byte base access is aligned for every group of 8 columns
  int32_t offs[kMaxSlices + 1];
  int32_t tile_start[kMaxSlices + 1];  // first column tile of each slice
  int32_t total_tiles;
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
  int bm, bn;        // gemm tile (tokens x stacked rank rows)
  int mf, nf;        // split-K kernel: row / column fragments of 16
  int mblocks, nblocks, ksplit;
  int64_t kps;
  int64_t partial_bytes;     // f32 partial tiles (0 unless ksplit > 1)
  int64_t grid;
};
// gemm_ok: the GEMM tiles may be chosen (their buffer loads address x and
// each slot's A block with 32-bit byte offsets).
ShrinkTiling choose_shrink_tiling(int64_t s, int64_t K, int CR, int num_segments, int chunk,
                                  bool gemm_ok = true);

struct ExpandTiling {
  int pairs, ks;     // 32-column fragment pairs per wave, 32-deep rank steps
  int64_t grid;
};

hipError_t launch_shrink(const ShrinkParams& p, const ShrinkTiling& t, hipStream_t stream);
hipError_t launch_shrink_gemm(const ShrinkParams& p, int bm, int bn, int64_t grid,
                              hipStream_t stream);
hipError_t launch_expand(const ExpandParams& p, const ExpandTiling& t, hipStream_t stream);
hipError_t launch_embedding(const EmbeddingParams& p, hipStream_t stream);

// The batch plan on the GPU (plan_device.hip): one workgroup; up to
// kDevicePlanMaxReqs requests and kDevicePlanMaxLoras slots.
constexpr int kDevicePlanMaxLoras = 1024;  // SGG_DEVICE_PLAN_MAX_LORAS
constexpr int kDevicePlanMaxReqs = 4096;   // SGG_DEVICE_PLAN_MAX_REQS
hipError_t launch_plan_device(const int32_t* seq_lens, const int32_t* req_slots, int32_t bs,
                              const int32_t* ranks, const float* scalings, int32_t L,
                              int32_t is_decode, int32_t max_chunk, int32_t chunk_override,
                              int64_t token_capacity, int32_t seg_capacity, const int64_t* off,
                              int32_t* plan, int32_t* info, hipStream_t stream);

// Copy n int32 from pinned host memory (given by its device-side address) to
// device memory, as a kernel on `stream`; src and dst 8-byte aligned.  When
// done_dev_view is not null (host memory, by its device-side address),
// done_value is written there once the source has been read in full.
hipError_t launch_plan_copy(const int32_t* src_dev_view, int32_t* dst, int64_t n,
                            int32_t* done_dev_view, int32_t done_value, hipStream_t stream);

}  // namespace sgg
