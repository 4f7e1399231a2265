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
  int64_t ldh, ldo, s, N;
  int32_t L, R, c, num_segments;
  int32_t vec8;               // 16-byte base access is aligned for every group of 8 columns
  int32_t offs[kMaxSlices + 1];
  int32_t tile_start[kMaxSlices + 1];  // first column tile of each slice
  int32_t total_tiles;
};

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
  int mf, nf;        // row / column fragments of 16
  int mblocks, nblocks, ksplit;
  int64_t kps;
  int64_t partial_bytes;     // f32 partial tiles (0 unless ksplit > 1)
  int64_t grid;
};
ShrinkTiling choose_shrink_tiling(int64_t s, int64_t K, int CR, int num_segments, int chunk);

struct ExpandTiling {
  int pairs, ks;     // 32-column fragment pairs per wave, 32-deep rank steps
  int64_t grid;
};

hipError_t launch_shrink(const ShrinkParams& p, const ShrinkTiling& t, hipStream_t stream);
hipError_t launch_expand(const ExpandParams& p, const ExpandTiling& t, hipStream_t stream);
hipError_t launch_embedding(const EmbeddingParams& p, hipStream_t stream);

}  // namespace sgg
