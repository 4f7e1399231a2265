// LoRA-A shrink: h[t, k*R + j] = sum_q A[a(t), k*R + j, q] * x[t, q] over the
// segments of a chunked plan (chunked_backend.py page: run_lora_a_sgemm and
// the shrink step of run_qkv_lora / run_gate_up_lora).
//
// One workgroup (4 waves) owns a tile of up to 16*MF tokens of one segment
// (gathered through the permutation) by 16*NF outputs of the c*R stacked
// rank rows, over one range of K.  The four waves take interleaved 64-deep K
// chunks of that range, each keeping the whole tile in its own MFMA
// accumulators, so no operand is fetched twice and the K loop needs no
// barrier; the four partial tiles are summed once through LDS at the end.
//
// Memory path.  An MFMA fragment puts 16 different rows on adjacent lanes, so
// loading fragments straight from row-major x / A costs one L1 access per
// lane.  Instead each chunk is fetched coalesced -- 8 lanes cover the 128
// contiguous bytes of one row, 8 rows per load -- into registers, written to
// the wave's own LDS tile, and read back in fragment layout.  Small tiles
// fetch several chunks per round trip (about 128 tile rows' worth), so a
// decode-sized K range is requested in one go.  Chunk slots in
// the LDS tile are XOR-swizzled by (row / 2) so that both the row-wise writes
// and the 16-row fragment reads hit 16 distinct bank groups.  The loads of
// chunk t+1 are in flight while chunk t is staged and multiplied; every load
// is unconditional (out-of-range rows / k read a clamped in-bounds address and
// are zeroed at the fragment read).
//
// When the segments alone cannot fill the GPU (decode batches) K is also
// split across workgroups: each writes an f32 partial tile and bumps an
// arrival counter; the last to arrive sums the partials in split order
// (deterministic) and writes bf16 h, then resets the counter.  In the
// stacked shrink + expand the partials are instead left for the expand,
// which sums them in the same order while staging h (no counters, no
// cross-workgroup round trip here).
#include "sgg_device.h"
#include "sgg_internal.h"
#include "sgg_kernels.h"

namespace sgg {

namespace {

constexpr int kFragsPerRound = 8;  // accumulator fragments reduced per LDS round

// Byte offset of 16-byte chunk c (0..7) of row r in a swizzled 128-byte-row tile.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

template <int MF, int NF>
__global__ __launch_bounds__(256, 1) void shrink_kernel(ShrinkParams p) {
  constexpr int BM = 16 * MF;
  constexpr int NB = 16 * NF;
  constexpr int NFR = MF * NF;
  constexpr int ROWS = BM + NB;          // tile rows per chunk: x rows, then A rows
  constexpr int LOADS = ROWS / 8;        // coalesced 16-byte loads per lane per chunk
  constexpr int XL = BM / 8;             // of which x rows
  constexpr int CH = ROWS >= 128 ? 1 : 128 / ROWS;  // chunks fetched per round trip
  constexpr int ROUNDS = (NFR + kFragsPerRound - 1) / kFragsPerRound;
  constexpr int STAGE_BYTES = 4 * CH * ROWS * 128;
  constexpr int RED_BYTES = 4 * kFragsPerRound * kWave * 16;
  __shared__ __attribute__((aligned(16))) char smem[STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES];
  __shared__ int last_flag;
  f32x4 (*red)[kFragsPerRound][kWave] = reinterpret_cast<f32x4 (*)[kFragsPerRound][kWave]>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  char* tile = smem + wave * CH * ROWS * 128;
  int seg, item;
  if (p.round_robin) {
    segment_round_robin(blockIdx.x, p.mblocks * p.nblocks * p.ksplit, &seg, &item);
    if (seg >= p.num_segments) return;
  } else {
    const int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int per = p.mblocks * p.nblocks * p.ksplit;
    seg = L / per;
    item = L % per;
  }
  const int mb0 = item % p.mblocks;
  const int nb = (item / p.mblocks) % p.nblocks;
  const int split = item / (p.mblocks * p.nblocks);

  // segment bounds, clamped to [0, s) so a malformed plan stays in bounds
  const int lo = max(p.seg_indptr[seg], 0);
  const int hi = min(static_cast<int64_t>(p.seg_indptr[seg + 1]), p.s);
  if (hi <= lo) return;
  const int slot = p.seg_slots[seg];
  int rho = (slot >= 0 && slot < p.L) ? p.ranks[slot] : 0;
  rho = rho < 0 ? 0 : (rho > p.R ? p.R : rho);
  const int a = rho > 0 ? slot : 0;
  if (rho == 0 && split != 0) return;  // split 0 alone writes the zero rows

  const int64_t kb = static_cast<int64_t>(split) * p.kps;
  const int64_t ke = kb + p.kps < p.K ? kb + p.kps : p.K;
  // this wave's 64-deep chunks: k = kb + 64*(wave + 4*t)
  const int64_t kw = kb + 64 * wave;
  const int nchunks = kw < ke ? static_cast<int>((ke - kw + 255) / 256) : 0;

  // Loading role of this lane: row (8*i + lane/8) of the chunk tile, 16-byte
  // piece lane%8 of the row's 128 bytes.
  const int lrow = lane >> 3;
  const int lcol = lane & 7;
  // Fragment role: row (lane%16) of a fragment, k group (lane/16).
  const int frow = lane & 15;
  const int fgrp = lane >> 4;

  // A rows of this lane's loads (fixed for the workgroup); rows beyond the
  // slot's rank or past c*R read row 0 of the slot (zeroed at the fragment read).
  const uint16_t* aslot = p.A + static_cast<int64_t>(a) * p.CR * p.K + 8 * lcol;
  int arow[LOADS - XL];
#pragma unroll
  for (int i = XL; i < LOADS; ++i) {
    const int n = nb * NB + (8 * i + lrow - BM);
    arow[i - XL] = (n < p.CR && (n % p.R) < rho) ? n : 0;
  }
  bool nvalid[NF];
#pragma unroll
  for (int g = 0; g < NF; ++g) {
    const int n = nb * NB + 16 * g + frow;
    nvalid[g] = n < p.CR && (n % p.R) < rho;
  }
  const uint16_t* xlane = p.x + 8 * lcol;

  for (int mb = mb0; lo + mb * BM < hi; mb += p.mblocks) {
    const int m0 = lo + mb * BM;
    const int mcount = hi - m0 < BM ? hi - m0 : BM;

    int xrow[XL];
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int mm = 8 * i + lrow;
      const int r = mm < mcount ? p.perm[m0 + mm] : 0;
      xrow[i] = (r >= 0 && r < p.s) ? r : 0;  // in-bounds stand-in, zeroed at the fragment read
    }
    bool tvalid[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      const int mm = 16 * f + frow;
      bool ok = mm < mcount;
      if (ok) {
        const int r = p.perm[m0 + mm];
        ok = r >= 0 && r < p.s;
      }
      tvalid[f] = ok;
    }

    f32x4 acc[NFR];
#pragma unroll
    for (int i = 0; i < NFR; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (rho > 0 && nchunks > 0) {
      // One register set of loads in flight: the CH chunks of stage t+1 are
      // requested as soon as stage t has been copied into the LDS tiles, and
      // arrive while stage t is multiplied.
      const int nstages = (nchunks + CH - 1) / CH;
      uint4 ld[CH][LOADS];
      auto issue = [&](int t) {
#pragma unroll
        for (int cc = 0; cc < CH; ++cc) {
          const int64_t k = kw + 256 * (CH * t + cc) + 8 * lcol;
          const int64_t koff = (k <= p.K - 8 ? k : p.K - 8) - 8 * lcol;
#pragma unroll
          for (int i = 0; i < XL; ++i)
            ld[cc][i] = load16(xlane + static_cast<int64_t>(xrow[i]) * p.ldx + koff);
#pragma unroll
          for (int i = XL; i < LOADS; ++i)
            ld[cc][i] = load16(aslot + static_cast<int64_t>(arow[i - XL]) * p.K + koff);
        }
      };
      issue(0);
      for (int t = 0; t < nstages; ++t) {
#pragma unroll
        for (int cc = 0; cc < CH; ++cc)
#pragma unroll
          for (int i = 0; i < LOADS; ++i)
            *reinterpret_cast<uint4*>(tile + cc * ROWS * 128 + swz(8 * i + lrow, lcol)) = ld[cc][i];
        if (t + 1 < nstages) issue(t + 1);
#pragma unroll
        for (int cc = 0; cc < CH; ++cc) {
          const int64_t k0 = kw + 256 * (CH * t + cc);
          if (k0 >= ke) break;  // wave-uniform
          const char* ct = tile + cc * ROWS * 128;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int c = 4 * st + fgrp;
            const bool kv = k0 + 8 * c < ke;
            uint4 xv[MF], av[NF];
#pragma unroll
            for (int f = 0; f < MF; ++f) {
              const uint4 v = *reinterpret_cast<const uint4*>(ct + swz(16 * f + frow, c));
              xv[f] = (kv && tvalid[f]) ? v : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int g = 0; g < NF; ++g) {
              const uint4 v = *reinterpret_cast<const uint4*>(ct + swz(BM + 16 * g + frow, c));
              av[g] = (kv && nvalid[g]) ? v : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int f = 0; f < MF; ++f)
#pragma unroll
              for (int g = 0; g < NF; ++g) acc[f * NF + g] = mfma16x16x32(av[g], xv[f], acc[f * NF + g]);
          }
        }
      }
    }

    // Sum the four waves' tiles through LDS, a few fragments per round, and
    // emit 4 consecutive outputs of one token per (fragment, lane) item.
    const bool direct = p.ksplit == 1 || rho == 0;
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      __syncthreads();
#pragma unroll
      for (int fr = 0; fr < kFragsPerRound; ++fr) {
        const int F = rd * kFragsPerRound + fr;
        if (F < NFR) red[wave][fr][lane] = acc[F];
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kFragsPerRound * kWave / 256; ++u) {
        const int q = tid + 256 * u;
        const int fr = q >> 6, l = q & 63;
        const int F = rd * kFragsPerRound + fr;
        if (F >= NFR) continue;
        const int f = F / NF, g = F % NF;
        const int mm = 16 * f + (l & 15);
        const int n = nb * NB + 16 * g + 4 * (l >> 4);
        if (mm >= mcount || n >= p.CR) continue;
        const f32x4 v = red[0][fr][l] + red[1][fr][l] + red[2][fr][l] + red[3][fr][l];
        if (direct) {
          const int r = p.perm[m0 + mm];
          if (r < 0 || r >= p.s) continue;
          uint2 o;
          o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
          o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
          *reinterpret_cast<uint2*>(p.h + static_cast<int64_t>(r) * p.ldh + n) = o;
        } else {
          // written through to the agent's coherence point (no dirty L2 lines)
          float* dst = p.partial + (static_cast<int64_t>(split) * p.s + (m0 + mm)) * p.CR + n;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __hip_atomic_store(dst + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if (direct || p.partials_only) continue;

    // Split-K: publish this partial, count arrivals, the last one reduces.
    // One release (thread 0, after the barrier that orders the whole
    // workgroup's partial stores before it) per workgroup, and one acquire
    // in the last arriver only: agent-scope fences write back / invalidate
    // the XCD's L2, so they are kept off every other path.
    __syncthreads();
    // (lo / BM + seg + mb) is distinct for every (segment, row block) of a
    // CSR plan, so every tile has its own counter; the clamp only keeps a
    // malformed plan in bounds.
    int64_t cidx = (static_cast<int64_t>(lo / BM) + seg + mb) * p.nblocks + nb;
    if (cidx >= p.counter_cap) cidx = p.counter_cap - 1;
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(p.counters + cidx, 1, __ATOMIC_RELEASE,
                                             __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == p.ksplit - 1;
      if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      last_flag = last;
    }
    __syncthreads();
    if (!last_flag) continue;
    const int items = mcount * (NB / 4);
    for (int q = tid; q < items; q += 256) {
      const int mm = q / (NB / 4);
      const int n = nb * NB + 4 * (q % (NB / 4));
      if (n >= p.CR) continue;
      const int r = p.perm[m0 + mm];
      if (r < 0 || r >= p.s) continue;
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int sp = 0; sp < p.ksplit; ++sp) {
        const float* src = p.partial + (static_cast<int64_t>(sp) * p.s + (m0 + mm)) * p.CR + n;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] += __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      uint2 o;
      o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(p.h + static_cast<int64_t>(r) * p.ldh + n) = o;
    }
    if (tid == 0) __hip_atomic_store(p.counters + cidx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int MF, int NF>
hipError_t launch_mn(const ShrinkParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((shrink_kernel<MF, NF>), dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <int MF>
hipError_t launch_m(const ShrinkParams& p, int nf, int64_t grid, hipStream_t stream) {
  switch (nf) {
    case 1: return launch_mn<MF, 1>(p, grid, stream);
    case 2: return launch_mn<MF, 2>(p, grid, stream);
    case 3: return launch_mn<MF, 3>(p, grid, stream);
    case 4: return launch_mn<MF, 4>(p, grid, stream);
    case 6: if constexpr (MF * 6 <= 32) return launch_mn<MF, 6>(p, grid, stream); break;
    case 8: if constexpr (MF * 8 <= 32) return launch_mn<MF, 8>(p, grid, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Tile choice.  Start from the largest tile (NF covering c*R up to 8
// fragments, MF covering the longest segment up to 8, at most 32 accumulator
// fragments per wave).  While the grid has fewer work items than CUs, split
// columns (NF), then rows (MF), down to single fragments; only then split K
// across workgroups, into at most 4 ranges (each extra range costs a partial
// tile round trip).  Measured on decode shapes: small tiles with 4 K ranges
// beat both one big tile and 16-32 K ranges.
ShrinkTiling choose_shrink_tiling(int64_t s, int64_t K, int CR, int num_segments, int chunk) {
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
  t.kps = (kgroups + ksplit - 1) / ksplit * 256;
  t.ksplit = static_cast<int>((K + t.kps - 1) / t.kps);
  if (t.ksplit < 1) t.ksplit = 1;
  t.grid = grid_for(num_segments, static_cast<int64_t>(t.ksplit) * t.nblocks * t.mblocks);
  if (t.ksplit > 1) t.partial_bytes = round_up(static_cast<int64_t>(t.ksplit) * s * CR * 4, 256);
  return t;
}

hipError_t launch_shrink(const ShrinkParams& p, const ShrinkTiling& t, hipStream_t stream) {
  if (t.grid <= 0) return hipSuccess;
  switch (t.mf) {
    case 1: return launch_m<1>(p, t.nf, t.grid, stream);
    case 2: return launch_m<2>(p, t.nf, t.grid, stream);
    case 4: return launch_m<4>(p, t.nf, t.grid, stream);
    case 8: return launch_m<8>(p, t.nf, t.grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sgg
