// Host-side tile choice for the LoRA-A shrink (the kernels are in shrink.hip
// and shrink_gemm.hip).  Plain host code: the launch code and the workspace
// size queries both call it, and the sanitizer build of the host code covers
// it without any device code.
#include "sgg_internal.h"
#include "sgg_kernels.h"

namespace sgg {

// Tile choice.  Batches that fill the GPU with whole-K tiles use the
// workgroup-shared GEMM kernel (shrink_gemm.hip); the rest use this kernel
// with K split.  For this kernel: start from the largest tile (NF covering c*R up to 8
// fragments, MF covering the longest segment up to 8, at most 32 accumulator
// fragments per wave).  While the grid has fewer work items than CUs, split
// columns (NF), then rows (MF), down to single fragments; only then split K
// across workgroups, into at most 4 ranges (each extra range costs a partial
// tile round trip).  Measured on decode shapes: small tiles with 4 K ranges
// beat both one big tile and 16-32 K ranges.  Grids that are already large
// enough take whole-K tiles, except batches of short segments with few rank
// rows and a long K, which take 64-token tiles with K split (below).
ShrinkTiling choose_shrink_tiling(int64_t s, int64_t K, int CR, int num_segments, int chunk,
                                  bool gemm_ok, bool pair_ok) {
  ShrinkTiling t{};
  static const int kNf[] = {1, 2, 3, 4, 6, 8};
  static const int kMf[] = {1, 2, 4, 8};
  const int need_n = (CR + 15) / 16;
  const int need_m = (chunk < 16 ? 16 : chunk + 15) / 16;
  // column fragments: values that tile c*R exactly (no partly empty block)
  auto nf_ok = [&](int v) { return v <= need_n ? need_n % v == 0 : v == kNf[0] || kNf[0] >= need_n; };
  int ni = 5, mi = 3;
  while (ni > 0 && (kNf[ni] > need_n && kNf[ni - 1] >= need_n)) --ni;  // smallest NF covering c*R
  while (ni > 0 && !(kNf[ni] >= need_n || need_n % kNf[ni] == 0)) --ni;
  while (mi > 0 && kMf[mi - 1] >= need_m) --mi;   // smallest MF covering the chunk (or 8)
  while (kMf[mi] * kNf[ni] > 32) --mi;
  auto units_for = [&](int nf, int mf) {
    const int bm = 16 * mf;
    const int64_t mblocks = (chunk + bm - 1) / bm;
    const int64_t grid_units = static_cast<int64_t>(num_segments) * mblocks;
    const int64_t real_units = (s + bm - 1) / bm + num_segments;
    const int64_t nblocks = (CR + 16 * nf - 1) / (16 * nf);
    return (grid_units < real_units ? grid_units : real_units) * nblocks;
  };
  while (units_for(kNf[ni], kMf[mi]) < 256 && ni > 0) {
    --ni;
    while (ni > 0 && !nf_ok(kNf[ni])) --ni;
  }
  while (units_for(kNf[ni], kMf[mi]) < 256 && mi > 0) --mi;
  t.nf = kNf[ni];
  t.mf = kMf[mi];
  t.nblocks = (CR + 16 * t.nf - 1) / (16 * t.nf);
  const int bm = 16 * t.mf;
  t.mblocks = (chunk + bm - 1) / bm;
  if (t.mblocks < 1) t.mblocks = 1;
  const int64_t units = units_for(t.nf, t.mf);
  const int64_t kgroups = (K + 255) / 256;   // 256-deep groups: one 64-deep chunk per wave
  int64_t ksplit = 1;
  const int64_t counters = (s / bm + num_segments + 1) * t.nblocks;
  if (units > 0 && units < 256 && counters <= kCounterCap) {
    ksplit = (256 + units - 1) / units;
    if (ksplit > 4) ksplit = 4;
    if (ksplit > kgroups) ksplit = kgroups;
  }
  // Tiles of 16 tokens over all the rank rows (33-48 of them: x read once
  // per K range instead of once per column block) with the fewest K ranges
  // (1, 2 or 4) that still give every CU a workgroup, for batches that had to
  // shrink their tiles to 16 tokens and whose segments hold 16 tokens or
  // more on average.  Measured on decode-shaped batches (stacked qkv, r = 16,
  // 8 adapters), stacked call: 1024 tokens 28.9 -> 25.9 us (K in 4), 2048
  // tokens 36.4 -> 31.5 us (K in 2).  Left out: 256 tokens (too few such
  // tiles: 10.1 vs 8.9 us), 4096 tokens (32-token tiles already fill the GPU;
  // such tiles 44.7-51 vs 42.6 us) and segments of a few tokens (decode over
  // 128 adapters: 35.0 vs 32.5 us).
  if (need_n == 3 && t.mf == 1 && t.nf < need_n &&
      s >= 16 * static_cast<int64_t>(num_segments)) {
    const int64_t u_all = units_for(need_n, 1);
    const int64_t c_all = s / 16 + num_segments + 1;
    for (int64_t ks : {int64_t{1}, int64_t{2}, int64_t{4}}) {
      if (ks > kgroups) break;
      if (u_all * ks >= 256 && (ks == 1 || c_all <= kCounterCap)) {
        t.nf = need_n;
        t.nblocks = 1;
        ksplit = ks;
        break;
      }
    }
  }
  t.kps = (kgroups + ksplit - 1) / ksplit * 256;
  t.ksplit = static_cast<int>((K + t.kps - 1) / t.kps);
  if (t.ksplit < 1) t.ksplit = 1;
  t.grid = grid_for(num_segments, static_cast<int64_t>(t.ksplit) * t.nblocks * t.mblocks);
  if (t.ksplit > 1) {
    t.partial_bytes = round_up(static_cast<int64_t>(t.ksplit) * s * CR * 4, 256);
    return t;
  }
  // No K split needed.  Batches of short segments whose stacked rank rows
  // are few (c*R <= 32) and that are small (at most 6144 tokens) or have a
  // long K (8192 or more) keep this kernel, with one K range and tiles of 32
  // tokens (64 above 6144 tokens) by half of c*R: its four waves stream
  // interleaved K chunks with no barrier between them.  Measured against the
  // 64 x 32 GEMM tiles (buffer loads, two register sets) on the full-layer
  // batch (4288 tokens, 93 segments, 64 adapters, r = 32): o_proj 22.7 vs
  // 25.6 us, down_proj 57.7 vs 65.2 us here; with c*R = 64 or more the GEMM
  // tiles win (qkv 39.1 -> 36.0 us, gate_up 33.2 -> 29.1 us, skewed
  // down_proj with r = 64: 149 -> 134 us).
  const bool long_segments = num_segments > 0 && s >= 96 * static_cast<int64_t>(num_segments);
  // With a long K (8192 or more) such batches fill the CUs from fewer
  // re-reads: tiles of 64 tokens by all of c*R (x read once, each A block
  // once per 64 tokens) with K split in ranges of 7 groups (1792): full-layer
  // down_proj (4288 tokens, 93 segments, K = 14336, r = 32) 77.7 -> 64.3 us,
  // against 66.0 us with K in 4, 70.1 us in 14 and 72.3 us with 128-token
  // tiles.  (On the skewed down_proj, c*R = 64, the GEMM tiles below stay
  // faster: 119 us against 176-212 us for such tiles.)
  if (!long_segments && CR <= 32 && K >= 8192) {
    const int nf = (CR + 15) / 16;
    const int64_t ranges = (kgroups + 6) / 7;
    const int64_t kps = (kgroups + ranges - 1) / ranges * 256;
    const int64_t nsplit = (K + kps - 1) / kps;
    const int64_t ncounters = s / 64 + num_segments + 1;   // one per 64-token tile
    const int64_t partial = round_up(nsplit * s * CR * 4, 256);
    if (nsplit > 1 && ncounters <= kCounterCap && partial < (int64_t{1} << 32) - 256) {
      t.mf = 4;
      t.nf = nf;
      t.nblocks = 1;
      t.mblocks = (chunk + 63) / 64;
      if (t.mblocks < 1) t.mblocks = 1;
      t.kps = kps;
      t.ksplit = static_cast<int>(nsplit);
      t.gemm = 0;
      t.grid = grid_for(num_segments, static_cast<int64_t>(t.ksplit) * t.mblocks);
      t.partial_bytes = partial;
      return t;
    }
  }
  if (!long_segments && CR <= 32 && (s <= 6144 || K >= 8192)) {
    t.mf = s > 6144 ? 4 : 2;
    t.nf = 1;
    for (int v : kNf)
      if (16 * v <= CR / 2 && t.mf * v <= 32) t.nf = v;
    t.nblocks = (CR + 16 * t.nf - 1) / (16 * t.nf);
    t.mblocks = (chunk + 16 * t.mf - 1) / (16 * t.mf);
    if (t.mblocks < 1) t.mblocks = 1;
    t.gemm = 0;
    t.grid = grid_for(num_segments, static_cast<int64_t>(t.nblocks) * t.mblocks);
    return t;
  }
  // The workgroup-shared GEMM tiles.  Batches of long
  // segments (mean work segment of 96 tokens or more, e.g. prefill) take
  // 128 tokens per tile and rank rows the smallest of 32 / 64 / 128 covering
  // c*R; batches of short segments (decode mixed in, many adapters, a long
  // tail of one-request adapters) take 64 x 32 tiles, whose larger grid
  // spreads the long segments over more CUs.  Then, while the grid has
  // fewer work items than CUs, halve the tokens if that alone fills the GPU
  // (x stays read once per column block; decode-shaped 16384 tokens, c*R =
  // 48: 64 x 64 tiles 48.9 us against 59.2 us for 128 x 32), else halve the
  // rows, then the tokens.  Measured: 64 x 32
  // beats 128 x 32 by 10-20 % on the mixed and skewed batches (full-layer
  // qkv 44 -> 39 us, skewed down_proj 202 -> 185 us), 128 x 128 beats every
  // smaller tile by 25 % or more on prefill; the split-K kernel is faster on
  // grids under one workgroup per CU.
  int gm = long_segments && chunk > 64 ? 128 : 64;
  int gn = !long_segments ? 32 : (CR <= 32 ? 32 : (CR <= 64 ? 64 : 128));
  auto gemm_units = [&](int m, int n) {
    const int64_t mb = (chunk + m - 1) / m, nbk = (CR + n - 1) / n;
    const int64_t grid_units = static_cast<int64_t>(num_segments) * mb;
    const int64_t real_units = (s + m - 1) / m + num_segments;
    return (grid_units < real_units ? grid_units : real_units) * nbk;
  };
  if (gemm_units(gm, gn) < 256 && gm > 64 && gemm_units(gm / 2, gn) >= 256) gm /= 2;
  while (gemm_units(gm, gn) < 256 && gn > 32) gn /= 2;
  while (gemm_units(gm, gn) < 256 && gm > 64) gm /= 2;
  // Too few workgroups for whole-K tiles (each workgroup has one K step of
  // loads in flight): the split-K kernel's finer tiles keep more CUs busy.
  if (gemm_units(gm, gn) < 256) return t;
  if (!gemm_ok) return t;  // x or an A block beyond 32-bit offsets: one K range here
  // Segment-pair tiles (only when asked for): for long segments with c*R
  // above 64, tiles of 256 tokens over pairs of consecutive work segments of
  // one slot, by 128 rank rows, with K split in two (f32 partials, summed in
  // split order).  Twice the tokens per read of the slot's A block cut the
  // L1 fill of the prefill gate_up shrink by a quarter (568 -> 433 MB), but
  // measured it is slower, 216 us against 94 us: at 96 KB of LDS and 356
  // registers a CU holds one such workgroup, the 284 workgroups run in two
  // rounds, and each CU fills at ~14 GB/s against ~21 GB/s for the 128 x 128
  // tiles.  (Splitting K of the 128 x 128 tiles alone, 544 workgroups,
  // measured 94 us: the fill, not the workgroup count, sets the time.)
  if (pair_ok && long_segments && gn == 128 && chunk <= 128 && kgroups >= 2) {
    const int64_t kps = (kgroups + 1) / 2 * 256;
    const int64_t ksplit = (K + kps - 1) / kps;
    const int64_t nblocks = (CR + 127) / 128;
    const int64_t counters = (s / 256 + num_segments + 1) * nblocks;
    const int64_t partial = round_up(ksplit * s * CR * 4, 256);
    if (ksplit >= 2 && counters <= kCounterCap && partial < (int64_t{1} << 32) - 256) {
      t.gemm = 1;
      t.bm = 256;
      t.bn = 128;
      t.kps = kps;
      t.ksplit = static_cast<int>(ksplit);
      t.mblocks = 1;
      t.nblocks = static_cast<int>(nblocks);
      t.partial_bytes = partial;
      t.grid = grid_for(num_segments, ksplit * nblocks);
      return t;
    }
  }
  t.gemm = 1;
  t.bm = gm;
  t.bn = gn;
  t.mblocks = (chunk + gm - 1) / gm;
  if (t.mblocks < 1) t.mblocks = 1;
  t.nblocks = (CR + gn - 1) / gn;
  t.grid = grid_for(num_segments, static_cast<int64_t>(t.nblocks) * t.mblocks);
  return t;
}

// The VALU form keeps the K split and the column tiles; only the token tiles
// shrink to 16 (so that a short segment's tile holds just its tokens).
void use_valu_tiles(ShrinkTiling* t, int64_t s, int num_segments, int chunk) {
  if (t->gemm || t->nf > 3 || t->grid <= 0) return;
  const int64_t counters = (s / 16 + num_segments + 1) * t->nblocks;
  if (t->ksplit > 1 && counters > kCounterCap) return;
  t->mf = 1;
  t->mblocks = chunk > 16 ? (chunk + 15) / 16 : 1;
  t->grid = grid_for(num_segments, static_cast<int64_t>(t->ksplit) * t->nblocks * t->mblocks);
  t->valu = 1;
}

// Producer tiling of the one-launch stacked call.  A decode batch's shrink is
// a chain of dependent memory round trips (plan, operands, partials) more
// than a stream of bytes, so the producers cover all c*R rank rows and up to
// 64 tokens each (x read once per K range, no cross-tile re-reads of A), and
// K is split as finely as the device can hold alongside the consumers: more
// ranges shorten each producer's load, at the price of more partials for the
// consumers to sum.
ShrinkTiling choose_fused_tiling(int64_t s, int64_t K, int CR, int num_segments, int chunk,
                                 int64_t consumers, int ks, int64_t resident, int force_ksplit) {
  ShrinkTiling t{};
  const int nf = (CR + 15) / 16;
  if (nf > 3 || num_segments <= 0 || s <= 0 || K <= 0) return t;
  const int64_t kgroups = (K + 255) / 256;
  // tallest tile that covers the longest segment first (no empty producers),
  // then shorter ones if its grid does not fit
  for (int mf : {4, 2, 1}) {
    if (mf > 1 && chunk <= 8 * mf) continue;   // a half-empty tile: take the next one
    const int64_t res = resident >= 0 ? resident : fused_resident_blocks(mf, nf, ks);
    const int64_t mblocks = (chunk + 16 * mf - 1) / (16 * mf);
    for (int want = kFusedMaxSplit; want >= 2; want /= 2) {   // partials need a split
      if (force_ksplit > 0 && want != force_ksplit) continue;
      const int64_t kps = (kgroups + want - 1) / want * 256;
      const int64_t ksplit = (K + kps - 1) / kps;
      const int64_t grid = grid_for(num_segments, mblocks * ksplit);
      if (ksplit < 2 || grid + consumers > res) continue;
      t.mf = mf;
      t.nf = nf;
      t.mblocks = static_cast<int>(mblocks < 1 ? 1 : mblocks);
      t.nblocks = 1;
      t.ksplit = static_cast<int>(ksplit);
      t.kps = kps;
      t.partial_bytes = round_up(ksplit * s * CR * 4, 256);
      t.grid = grid;
      return t;
    }
  }
  return t;
}

}  // namespace sgg
