// LoRA-B expand work item (one column tile of one segment) and its block
// mapping.  The algorithm is described at the top of expand.hip.
#pragma once

#include "sgg_device.h"
#include "sgg_kernels.h"

namespace sgg {
namespace detail {

template <int P, int KS>
struct ExpandShape {
  static constexpr int TNW = 32 * P;                  // columns per wave
  static constexpr int CPR = 4 * KS;                  // 16-byte chunks per LDS h row (R <= 32*KS)
  static constexpr int RPS = 16 / CPR > 0 ? 16 / CPR : 1;  // h rows sharing one swizzle value
  static constexpr int LPR = 4 * P;                   // lanes per base row segment (16 B each)
  static constexpr int RPL = 64 / LPR;                // base rows per wave load
  static constexpr int BLD = 16 / RPL;                // base loads per 16 tokens
  static constexpr int APAD = TNW + 4;                // floats per row of the transpose tile
  static constexpr int HTILE_BYTES = 128 * CPR * 16;
  static constexpr int PROW_BYTES = 128 * 4;
  static constexpr int ACCT_BYTES = 4 * 16 * APAD * 4;
  static constexpr int SMEM = HTILE_BYTES + PROW_BYTES + ACCT_BYTES;
};

// No hand-off: h (or the partials) was written by an earlier launch.
struct NoWait {
  __device__ __forceinline__ bool operator()() const { return false; }
};

// Work item of block b: false for the padding blocks of the grid.
//
// Column tiles dealt to the XCDs (tiles_per_xcd > 0): block b runs on XCD
// x = b % 8 and takes tile x + 8*j of segment seg, walking its share of the
// tiles of segment 0, then of segment 1, and so on.  Each XCD thus needs only
// one eighth of an adapter's B columns, and reuses them from its L2 across
// the adapter's consecutive segments while they are hot; every XCD gets an
// equal share of every segment, however the tokens fall on the adapters; the
// h rows of a segment are read by all eight XCDs (they are a small fraction
// of the bytes).  Otherwise segments are dealt to the XCDs
// (segment_round_robin): all tiles of a segment on one XCD.
__device__ __forceinline__ bool expand_item_of(const ExpandParams& p, int b, int* seg, int* tile) {
  if (p.tiles_per_xcd > 0) {
    const int x = b % kXcds, l = b / kXcds;
    *seg = l / p.tiles_per_xcd;
    *tile = (l % p.tiles_per_xcd) * kXcds + x;
    return *seg < p.num_segments && *tile < p.total_tiles;
  }
  segment_round_robin(b, p.total_tiles, seg, tile);
  return *seg < p.num_segments;
}

// Column tile `tile` of segment `seg`; `smem` holds ExpandShape<P, KS>::SMEM
// bytes (16-byte aligned).  `wait()` runs once, by the whole workgroup, after
// the B fragments are requested and before h is staged (the fused launch
// waits there for its segment's partials; it may use `smem`).  It returns
// true when it did other work meanwhile, and the B fragments are then
// requested again rather than held across it.
// HPART: h comes as split-K partials (p.hpart), else as bf16 rows (p.h); a
// template flag, so an instance carries only the staging code it runs (the
// other path's loads otherwise cost the main loop its wait counts).
template <int P, int KS, bool HPART, bool FUSED = false, class Wait = NoWait>
__device__ __forceinline__ void expand_tile(const ExpandParams& p, int seg, int tile, char* smem,
                                            const Wait& wait = Wait()) {
  using S = ExpandShape<P, KS>;
  constexpr int TNW = S::TNW;
  constexpr int CPR = S::CPR;
  constexpr int RPS = S::RPS;
  constexpr int LPR = S::LPR;
  constexpr int RPL = S::RPL;
  constexpr int BLD = S::BLD;
  constexpr int APAD = S::APAD;
  uint4* htile = reinterpret_cast<uint4*>(smem);
  int* prow = reinterpret_cast<int*>(smem + S::HTILE_BYTES);
  float (*acct)[16 * APAD] =
      reinterpret_cast<float (*)[16 * APAD]>(smem + S::HTILE_BYTES + S::PROW_BYTES);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int k = 0;
  while (k + 1 < p.c && tile >= p.tile_start[k + 1]) ++k;
  const int colt = p.offs[k] + (tile - p.tile_start[k]) * (128 * P);
  const int colw = colt + TNW * wave;
  const int colend = p.offs[k + 1];

  // segment bounds, clamped to [0, s) so a malformed plan stays in bounds
  const int lo = max(p.seg_indptr[seg], 0);
  const int hi = min(static_cast<int64_t>(p.seg_indptr[seg + 1]), p.s);
  if (hi <= lo || colt >= colend) return;
  const int slot = p.seg_slots[seg];
  const bool slot_ok = slot >= 0 && slot < p.L;
  const bool active = colw < colend;  // wave has columns (uniform); keeps joining barriers
  const int m = lane & 15;
  const int q = lane >> 4;

  // B fragments: fragment g row m is column colw + 16*g + m; rank chunk 8q + 32ks.
  // With one rank step (R <= 32) they are requested before the slot's rank
  // arrives (every column j < R is in bounds) and columns at or beyond the
  // rank are zeroed once it is known.  With more rank steps only the chunks
  // below the rank are requested, after it arrives: padded ranks then cost
  // no B bytes (skewed batch, ranks 8-64 padded to 64: expands 55.5 ->
  // 52.5 us; prefill unchanged).
  uint4 bw[2 * P][KS];
  const auto load_b = [&](int jmax) {
#pragma unroll
    for (int g = 0; g < 2 * P; ++g) {
      const int n = colw + 16 * g + m;
      const uint16_t* brow =
          p.B + (static_cast<int64_t>(slot_ok ? slot : 0) * p.N + (n < colend ? n : 0)) * p.R;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int j = 32 * ks + 8 * q;
        bw[g][ks] = make_uint4(0, 0, 0, 0);
        if (active && n < colend && j < jmax) bw[g][ks] = load16(brow + j);
      }
    }
  };
  constexpr bool kRankAwareB = KS >= 2 && !FUSED;
  if constexpr (!kRankAwareB) load_b(p.R);
  int rho = slot_ok ? p.ranks[slot] : 0;
  rho = rho < 0 ? 0 : (rho > p.R ? p.R : rho);
  if (rho == 0) return;  // base model: output rows stay untouched
  if constexpr (kRankAwareB) load_b(rho);
  const float sigma = p.scalings[slot];
  // Base-row role of this lane: row (RPL*i + lane/LPR) of a 16-token group,
  // columns colw + 8*(lane%LPR) .. +7.
  const int brw = lane / LPR;
  const int bc = colw + 8 * (lane % LPR);
  const bool bvec = p.vec8 && bc + 8 <= colend;
  // FUSED: the base rows of the first two 16-token groups are requested
  // before the wait, so they arrive while the shrink tiles run.
  uint4 pre[2][BLD];
  const auto prefetch = [&]() {
    const int ntok0 = hi - lo < 128 ? hi - lo : 128;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int i = 0; i < BLD; ++i) {
        const int rr = 16 * f + RPL * i + brw;
        int r = rr < ntok0 ? p.perm[lo + rr] : -1;
        r = (r >= 0 && r < p.s) ? r : -1;
        pre[f][i] = make_uint4(0, 0, 0, 0);
        if (r >= 0 && bvec && active)
          pre[f][i] = *reinterpret_cast<const uint4*>(p.out + static_cast<int64_t>(r) * p.ldo + bc);
      }
  };
  if constexpr (FUSED) prefetch();
  if (wait()) {  // fragments and rows are in flight during a plain wait
    load_b(p.R);
    if constexpr (FUSED) prefetch();
  }
  // The B fragments are masked to the rank just before their first use, so
  // their loads stay in flight while h is staged.
  bool b_masked = false;

  const int hch = p.R >> 3;  // 16-byte chunks of one h row slice
  float* at = acct[wave];

  for (int c0 = lo; c0 < hi; c0 += 128) {
    const int ntok = hi - c0 < 128 ? hi - c0 : 128;
    __syncthreads();  // previous chunk's tiles are no longer read
    if (tid < ntok) {
      const int r = p.perm[c0 + tid];
      prow[tid] = (r >= 0 && r < p.s) ? r : -1;
    }
    if constexpr (HPART) {
      // Split-K partials, indexed by sorted position (no gather): each
      // (row, 8-column chunk) sums its splits in split order, with the loads
      // of several splits in flight at a time, and rounds the sum to bf16 into
      // the h tile.  Partials written by an earlier launch are read through
      // the caches; in the one-launch form they come from other workgroups of
      // the same launch, so they are read device-coherently.
      const __amdgpu_buffer_rsrc_t prsrc = buffer_rsrc(p.hpart, p.hpart_bytes);
      const auto part16 = [&](int64_t idx) {
        if constexpr (FUSED) return load_coherent16(prsrc, static_cast<uint32_t>(idx * 4));
        else return *reinterpret_cast<const f32x4*>(p.hpart + idx);
      };
      const int64_t split_stride = p.s * p.ldp;
      for (int piece = tid; piece < ntok * hch; piece += 256) {
        const int row = piece / hch, c = piece % hch;
        const int64_t src = static_cast<int64_t>(c0 + row) * p.ldp + k * p.R + 8 * c;
        f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
        int sp = 0;
        // Splits whose loads are in flight together: four, except in the
        // 256-column tiles with one rank step, where two keep the kernel at
        // 92 registers and five workgroups per CU instead of 108 and four
        // (MoE add 33.9 -> 30.5 us; the sums keep the same order).
        constexpr int SB = (P == 2 && KS == 1) ? 2 : 4;
        for (; sp + SB <= p.hsplit; sp += SB) {
          f32x4 lo4[SB], hi4[SB];
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            lo4[u] = part16(src + (sp + u) * split_stride);
            hi4[u] = part16(src + (sp + u) * split_stride + 4);
          }
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            s0 += lo4[u];
            s1 += hi4[u];
          }
        }
        for (; sp < p.hsplit; ++sp) {
          s0 += part16(src + sp * split_stride);
          s1 += part16(src + sp * split_stride + 4);
        }
        uint4 v;
        v.x = f32_to_bf16(s0[0]) | (f32_to_bf16(s0[1]) << 16);
        v.y = f32_to_bf16(s0[2]) | (f32_to_bf16(s0[3]) << 16);
        v.z = f32_to_bf16(s1[0]) | (f32_to_bf16(s1[1]) << 16);
        v.w = f32_to_bf16(s1[2]) | (f32_to_bf16(s1[3]) << 16);
        htile[row * CPR + (c ^ ((row / RPS) % CPR))] = v;
      }
    } else {
      for (int piece = tid; piece < ntok * hch; piece += 256) {
        const int row = piece / hch, c = piece % hch;
        const int r = p.perm[c0 + row];
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r >= 0 && r < p.s) v = load16(p.h + static_cast<int64_t>(r) * p.ldh + k * p.R + 8 * c);
        htile[row * CPR + (c ^ ((row / RPS) % CPR))] = v;
      }
    }
    __syncthreads();
    if (!active) continue;

    const int nf = (ntok + 15) >> 4;
    uint4 bv0[BLD], bv1[BLD];
    auto fetch = [&](int f, uint4 (&bv)[BLD]) {
#pragma unroll
      for (int i = 0; i < BLD; ++i) {
        const int rr = 16 * f + RPL * i + brw;
        const int r = rr < ntok ? prow[rr] : -1;
        bv[i] = make_uint4(0, 0, 0, 0);
        if (r >= 0 && bvec)
          bv[i] = *reinterpret_cast<const uint4*>(p.out + static_cast<int64_t>(r) * p.ldo + bc);
      }
    };
    auto step = [&](int f, const uint4 (&bv)[BLD]) {
      // h fragment: row 16f + m, rank chunk 8q + 32ks
      const int hr = 16 * f + m;
      const bool hv_ok = hr < ntok && prow[hr] >= 0;
      uint4 hv[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int j = 32 * ks + 8 * q;
        const int c = 4 * ks + q;
        hv[ks] = make_uint4(0, 0, 0, 0);
        if (hv_ok && j < rho) hv[ks] = keep_first(htile[hr * CPR + (c ^ ((hr / RPS) % CPR))], rho - j);
      }
#pragma unroll
      for (int g = 0; g < 2 * P; ++g) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(bw[g][ks], hv[ks], acc);
        *reinterpret_cast<f32x4*>(at + m * APAD + 16 * g + 4 * q) = acc;
      }
      // transposed read: 8 consecutive columns of one token per lane
#pragma unroll
      for (int i = 0; i < BLD; ++i) {
        const int rl = RPL * i + brw;
        const int rr = 16 * f + rl;
        const int r = rr < ntok ? prow[rr] : -1;
        if (r < 0 || bc >= colend) continue;
        const float* src = at + rl * APAD + 8 * (lane % LPR);
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(src + 4);
        uint16_t* dst = p.out + static_cast<int64_t>(r) * p.ldo + bc;
        if (bvec) {
          const uint4 b = bv[i];
          uint4 o;
          o.x = f32_to_bf16(bf16_to_f32(b.x & 0xffffu) + sigma * a0[0]) |
                (f32_to_bf16(bf16_to_f32(b.x >> 16) + sigma * a0[1]) << 16);
          o.y = f32_to_bf16(bf16_to_f32(b.y & 0xffffu) + sigma * a0[2]) |
                (f32_to_bf16(bf16_to_f32(b.y >> 16) + sigma * a0[3]) << 16);
          o.z = f32_to_bf16(bf16_to_f32(b.z & 0xffffu) + sigma * a1[0]) |
                (f32_to_bf16(bf16_to_f32(b.z >> 16) + sigma * a1[1]) << 16);
          o.w = f32_to_bf16(bf16_to_f32(b.w & 0xffffu) + sigma * a1[2]) |
                (f32_to_bf16(bf16_to_f32(b.w >> 16) + sigma * a1[3]) << 16);
          *reinterpret_cast<uint4*>(dst) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (bc + e < colend) {
              const float v = e < 4 ? a0[e & 3] : a1[e & 3];
              const float y = bf16_to_f32(dst[e]) + sigma * v;
              dst[e] = static_cast<uint16_t>(f32_to_bf16(y));
            }
          }
        }
      }
    };
    if (!b_masked) {
#pragma unroll
      for (int g = 0; g < 2 * P; ++g)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bw[g][ks] = keep_first(bw[g][ks], rho - (32 * ks + 8 * q));
      b_masked = true;
    }
    const bool use_pre = FUSED && c0 == lo;
    if (use_pre) {
#pragma unroll
      for (int i = 0; i < BLD; ++i) bv0[i] = pre[0][i];
    } else {
      fetch(0, bv0);
    }
    for (int f = 0; f < nf; f += 2) {
      if (f + 1 < nf) {
        if (use_pre && f == 0) {
#pragma unroll
          for (int i = 0; i < BLD; ++i) bv1[i] = pre[1][i];
        } else {
          fetch(f + 1, bv1);
        }
      }
      step(f, bv0);
      if (f + 1 < nf) {
        if (f + 2 < nf) fetch(f + 2, bv0);
        step(f + 1, bv1);
      }
    }
  }
}

}  // namespace detail
}  // namespace sgg
