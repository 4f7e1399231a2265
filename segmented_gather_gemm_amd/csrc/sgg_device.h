// Device-side helpers for the gfx950 kernels: bf16 bit handling, 16-byte
// fragment loads, the MFMA operand types and the XCD-aware block mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sgg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// 8 bf16 values (16 bytes) from a 16-byte aligned address.
__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Zero the elements at positions >= keep (keep in any range) of 8 packed bf16.
__device__ __forceinline__ uint4 keep_first(uint4 v, int keep) {
  if (keep >= 8) return v;
  if (keep <= 0) return make_uint4(0, 0, 0, 0);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int lo = 2 * i, hi = 2 * i + 1;
    uint32_t m = (lo < keep ? 0x0000ffffu : 0u) | (hi < keep ? 0xffff0000u : 0u);
    w[i] &= m;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// D (16x16, f32) += A (16x32) * B (32x16), bf16 inputs.  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, each with the 8 consecutive k of
// group (l / 16); it receives D rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Raw buffer resource over `bytes` bytes at `base` (32-bit data format):
// loads at or past the end return zero and stores there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// 16 bytes at byte offset `off` of a buffer, with device-scope coherence
// (the sc1 cache policy: the access sees, and is seen by, the other
// workgroups of the device -- what an agent-scope atomic access does, 16
// bytes at a time and without waiting for each access).
constexpr int kDeviceScopePolicy = 16;
__device__ __forceinline__ f32x4 load_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       r, static_cast<int>(off), 0, kDeviceScopePolicy));
}
__device__ __forceinline__ void store_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                 f32x4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r,
                                         static_cast<int>(off), 0, kDeviceScopePolicy);
}

// Wait until this wave's outstanding vector memory operations have completed
// (also a compiler memory barrier).  Cross-workgroup hand-offs publish data
// with device-coherent stores (store_coherent16), which write through to the
// point of coherence of the whole device; once every wave of the workgroup
// has waited for its own stores, a barrier and one counter RMW make the data
// safe to read with device-coherent loads from any XCD.  No L2 write-back (release) or
// invalidate (acquire) is needed for data moved that way, and both are
// costly here: a write-back per wave doubled the decode shrink's time.
__device__ __forceinline__ void wave_stores_done() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Blocks are handed to the XCDs round-robin (block b runs on XCD b % 8).
// Segments are dealt round-robin to the XCDs the same way: block b takes
// segment (b % 8) + 8 * ((b / 8) / per) and item (b / 8) % per of it, so the
// items of one segment share an XCD (and its L2), while consecutive segments
// -- the full chunks of a dominant adapter, or the real segments ahead of a
// graph's capacity padding -- spread over all XCDs.  Measured against
// dealing groups of consecutive segments (up to one contiguous range per
// XCD): single segments are as fast or faster on every workload, and with
// one adapter holding most tokens contiguous ranges make the expand take
// 1.7x as long, its full chunks crowding onto two or three XCDs.
// Launch with grid_for(num_segments, per) blocks.
__device__ __forceinline__ void segment_round_robin(int b, int per, int* seg, int* item) {
  const int x = b % kXcds, l = b / kXcds;
  *seg = x + kXcds * (l / per);
  *item = l % per;
}

// MoE routing (PR #24007 report page, implementation breakdown items 2-4):
// the virtual expert a(t) * E + topk_ids[m] of top-k copy m of token
// t = m / top_k, where a(t) is the slot of the request r with
// req_seg_indptr[r] <= t < req_seg_indptr[r + 1] -- request t itself when it
// holds the token (one-token requests: one round trip), else found by binary
// search.  A copy whose request, adapter or expert is out of range goes to
// the extra virtual slot L * E.
__device__ __forceinline__ int moe_virtual_slot(const int32_t* req_seg_indptr,
                                                const int32_t* req_weight_indices, int bs,
                                                const int32_t* topk_ids, int top_k, int E, int L,
                                                int64_t m) {
  const int64_t t = m / top_k;
  const int e = topk_ids[m];
  int r = -1;
  if (t < bs && req_seg_indptr[t] <= t && t < req_seg_indptr[t + 1]) {
    r = static_cast<int>(t);
  } else {
    int lo = 0, hi = bs;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (req_seg_indptr[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    if (lo < bs && req_seg_indptr[lo] <= t && t < req_seg_indptr[lo + 1]) r = lo;
  }
  int v = L * E;
  if (r >= 0) {
    const int a = req_weight_indices[r];
    if (a >= 0 && a < L && e >= 0 && e < E) v = a * E + e;
  }
  return v;
}

}  // namespace sgg
