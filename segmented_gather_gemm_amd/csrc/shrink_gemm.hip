// LoRA-A shrink for batches that fill the GPU without splitting K (prefill,
// mixed batches): h[t, k*R + j] = sum_q A[a(t), k*R + j, q] * x[t, q] over
// the segments of a plan (chunked_backend.py page: run_lora_a_sgemm and the
// shrink step of run_qkv_lora / run_gate_up_lora).
//
// A workgroup (4 waves) owns BM gathered tokens of one segment by BN stacked
// rank rows and walks K in 64-deep steps.  Each step's x rows and A rows are
// fetched once for the whole workgroup -- coalesced, 8 lanes per 128-byte
// row -- into one of two XOR-swizzled LDS stages; every wave then reads its
// (BM / WM) x (BN / WN) share of the tile as MFMA fragments
// (mfma_f32_16x16x32_bf16).  The next step's loads are in flight while the
// current step is multiplied, and one barrier per step separates the two.
//
// No operand is masked inside the K loop: a token row outside the segment
// (or with an invalid permutation entry) reads an in-bounds stand-in row and
// only feeds its own output row, which is never stored; an A row beyond the
// slot's rank (or beyond c*R) reads the slot's row 0 instead of its padding
// and only feeds its own output column, which is stored as zero.  A tile
// whose rank rows all lie past the slot's rank writes zeros and skips the K
// loop.  Only a ragged K tail (K % 64 != 0) zeroes the chunks past K, in its
// last step.
//
// x and the slot's A block are read with buffer loads: a per-lane 32-bit row
// offset fixed for the workgroup plus the step's K offset in a scalar
// register, so the K loop spends no vector registers or instructions on
// addresses, and a read past the end of the buffer returns zero instead of
// faulting.  The host takes this kernel only when x and every slot's A block
// fit in 4 GiB of offsets.
//
// With two or more register sets, every step requests the loads of step
// t + DEPTH unconditionally (the last step again once past the end) and the
// ragged-K zeroing happens while staging: a load issued under a branch makes
// the compiler's wait before staging step t + 1 count conservatively and
// drain the newer sets too (s_waitcnt vmcnt(0)), which serialises the
// pipeline.  Measured on the skewed o_proj batch (64 x 32 tiles): 42 -> 35
// us.  With one register set the branchy form is faster (prefill 128 x 128
// tiles: 97 us against 122 us).
#include "sgg_device.h"
#include "sgg_kernels.h"
#include "shrink_tile.h"

namespace sgg {

namespace {

// Byte offset of 16-byte chunk c (0..7) of row r in a swizzled 128-byte-row tile.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

// Fourth word of a raw buffer resource on gfx9 (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

// 16 bytes at byte offset voff + soff of a buffer (soff uniform).
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                               int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                       rsrc, static_cast<int>(voff), soff, 0));
}

template <int BM, int BN, int WM, int DEPTH, bool PAIR = false>
__global__ __launch_bounds__(256, PAIR ? 1 : 2) void shrink_gemm_kernel(ShrinkParams p) {
  constexpr int WN = 4 / WM;
  constexpr int FM = BM / (16 * WM);        // token fragments per wave
  constexpr int FN = BN / (16 * WN);        // rank-row fragments per wave
  constexpr int ROWS = BM + BN;             // tile rows per step: x rows, then A rows
  constexpr int XPER = BM / 32;             // 16-byte loads per thread per step: x rows
  constexpr int APER = BN / 32;             //   and A rows
  constexpr int STAGE = ROWS * 128;         // bytes of one LDS stage
  static_assert(FM >= 1 && FN >= 1 && ROWS % 32 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  int seg, item;
  segment_round_robin(blockIdx.x, p.mblocks * p.nblocks * (PAIR ? p.ksplit : 1), &seg, &item);
  if (seg >= p.num_segments) return;
  int split = 0;
  if constexpr (PAIR) {
    split = item / (p.mblocks * p.nblocks);
    item %= p.mblocks * p.nblocks;
  }
  const int mb0 = item % p.mblocks;
  const int nb = item / p.mblocks;
  const int slot = p.seg_slots[seg];
  // segment bounds, clamped to [0, s) so a malformed plan stays in bounds
  const int lo = max(p.seg_indptr[seg], 0);
  int64_t end = p.seg_indptr[seg + 1];
  if constexpr (PAIR) {
    // Tiles over pairs (2i, 2i+1) of consecutive segments of one slot (a
    // contiguous range of sorted positions); the odd one of a pair exits.
    if (seg & 1) {
      if (p.seg_slots[seg - 1] == slot) return;
    } else if (seg + 1 < p.num_segments && p.seg_slots[seg + 1] == slot) {
      end = p.seg_indptr[seg + 2];
    }
  }
  const int hi = min(end, p.s);
  if (hi <= lo) return;
  const bool slot_ok = slot >= 0 && slot < p.L;
  int rho = slot_ok ? p.ranks[slot] : 0;
  rho = rho < 0 ? 0 : (rho > p.R ? p.R : rho);

  // Loading role: row (tid/8 + 32*j) of the step's tile, 16-byte chunk tid%8.
  const int lrow = tid >> 3;
  const int lcol = tid & 7;
  // Raw buffer resources over the slot's A block and over x (loads at or past
  // the end of a range return zero).
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.A + static_cast<int64_t>(slot_ok ? slot : 0) * p.CR * p.K),
      static_cast<short>(0), static_cast<int>(static_cast<uint32_t>(p.CR * p.K * 2)), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.x), static_cast<short>(0),
      static_cast<int>(static_cast<uint32_t>(((p.x_rows - 1) * p.ldx + p.K) * 2)), kRsrcWord3);
  // A rows of this thread's loads (tile rows BM + lrow + 32*j), fixed for the
  // workgroup.  Rows past c*R or past the slot's rank (padding, possibly NaN)
  // read row 0 of the slot instead, a live row that stays in L1: their
  // products only reach output rows stored as zero, and the L1 fill is spent
  // on live rows.
  uint32_t aoff[APER];
#pragma unroll
  for (int j = 0; j < APER; ++j) {
    const int n = nb * BN + lrow + 32 * j;
    const bool live = n < p.CR && (n % p.R) < rho;
    aoff[j] = static_cast<uint32_t>((live ? n : 0) * p.K * 2 + 16 * lcol);
  }
  // Whether any rank row of this tile lies within the slot's rank (uniform):
  // a tile of padding rows only writes zeros and reads nothing.
  bool tile_live = false;
  {
    const int n0 = nb * BN, n1 = min(n0 + BN, p.CR);
    for (int k = n0 / p.R; k * p.R < n1 && !tile_live; ++k)
      tile_live = max(n0, k * p.R) - k * p.R < rho;
  }
  // 64-deep K steps [kt0, kt0 + nk) of this workgroup (PAIR: split `split`
  // of p.ksplit ranges of p.kps)
  const int nk_all = static_cast<int>((p.K + 63) / 64);
  int kt0 = 0, nk = nk_all;
  if constexpr (PAIR) {
    const int per = static_cast<int>(p.kps / 64);
    kt0 = split * per;
    nk = nk_all - kt0 < per ? nk_all - kt0 : per;
  }
  const bool ktail = (p.K & 63) != 0;
  const bool dead = rho == 0 || !tile_live;
  if (PAIR && dead && split != 0) return;  // split 0 alone writes the zero rows

  // Fragment role: row (lane%16) of a fragment, k group (lane/16).
  const int frow = lane & 15;
  const int fgrp = lane >> 4;
  const int xr0 = wm * FM * 16;             // this wave's first token row in the tile
  const int ar0 = BM + wn * FN * 16;        // this wave's first A row in the tile

  for (int mb = mb0; lo + mb * BM < hi; mb += p.mblocks) {
    const int m0 = lo + mb * BM;
    const int mcount = hi - m0 < BM ? hi - m0 : BM;

    if (dead) {  // base model slot or padding rows: zero rows of h
      for (int q = tid; q < mcount * (BN / 4); q += 256) {
        const int mm = q / (BN / 4);
        const int n = nb * BN + 4 * (q % (BN / 4));
        const int r = p.perm[m0 + mm];
        if (n < p.CR && r >= 0 && r < p.s)
          *reinterpret_cast<uint2*>(p.h + static_cast<int64_t>(r) * p.ldh + n) = make_uint2(0, 0);
      }
      continue;
    }

    // x rows of this thread's loads (tile rows lrow + 32*j; a stand-in row
    // for tokens outside the segment)
    uint32_t xoff[XPER];
#pragma unroll
    for (int j = 0; j < XPER; ++j) {
      const int r = lrow + 32 * j;
      const int pr = r < mcount ? p.perm[m0 + r] : p.perm[m0];
      const int xr = (pr >= 0 && pr < p.s) ? (p.xdiv > 1 ? pr / p.xdiv : pr) : 0;
      xoff[j] = static_cast<uint32_t>(static_cast<int64_t>(xr) * p.ldx * 2 + 16 * lcol);
    }

    // DEPTH register sets of prefetch: step t + DEPTH is requested while
    // step t is multiplied from LDS stage t & 1 and step t + 1, requested
    // DEPTH - 1 steps earlier, waits in its register set to be staged.  The
    // loop is unrolled by DEPTH so that each register set is a fixed one.
    uint4 xl[DEPTH][XPER], al[DEPTH][APER];
    // chunk lcol of step kt lies past a ragged end of K: it contributes zero
    auto past_k = [&](int kt) {
      return ktail && kt0 + kt == nk_all - 1 &&
             static_cast<int64_t>(kt0 + kt) * 64 + 8 * lcol >= p.K;
    };
    auto issue = [&](int kt, uint4 (&xs)[XPER], uint4 (&as)[APER]) {
      const int soff = (kt0 + kt) * 128;
#pragma unroll
      for (int j = 0; j < XPER; ++j) xs[j] = buffer_load16(xrsrc, xoff[j], soff);
#pragma unroll
      for (int j = 0; j < APER; ++j) as[j] = buffer_load16(arsrc, aoff[j], soff);
      if constexpr (DEPTH == 1) {
        if (past_k(kt)) {
#pragma unroll
          for (int j = 0; j < XPER; ++j) xs[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < APER; ++j) as[j] = make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto stash = [&](int buf, int kt, const uint4 (&xs)[XPER], const uint4 (&as)[APER]) {
      char* st = smem + buf * STAGE;
      const bool kill = DEPTH > 1 && past_k(kt);
#pragma unroll
      for (int j = 0; j < XPER; ++j)
        *reinterpret_cast<uint4*>(st + swz(lrow + 32 * j, lcol)) =
            kill ? make_uint4(0, 0, 0, 0) : xs[j];
#pragma unroll
      for (int j = 0; j < APER; ++j)
        *reinterpret_cast<uint4*>(st + swz(BM + lrow + 32 * j, lcol)) =
            kill ? make_uint4(0, 0, 0, 0) : as[j];
    };
    auto mma = [&](int buf, f32x4 (&acc)[FN][FM]) {
      const char* st = smem + buf * STAGE;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = 4 * ks + fgrp;
        uint4 xv[FM], av[FN];
#pragma unroll
        for (int f = 0; f < FM; ++f)
          xv[f] = *reinterpret_cast<const uint4*>(st + swz(xr0 + 16 * f + frow, c));
#pragma unroll
        for (int i = 0; i < FN; ++i)
          av[i] = *reinterpret_cast<const uint4*>(st + swz(ar0 + 16 * i + frow, c));
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int f = 0; f < FM; ++f) acc[i][f] = mfma16x16x32(av[i], xv[f], acc[i][f]);
      }
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int f = 0; f < FM; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // the previous row block's tiles are no longer read
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      if constexpr (DEPTH == 1) {
        if (u < nk) issue(u, xl[u], al[u]);
      } else {
        issue(u < nk ? u : nk - 1, xl[u], al[u]);
      }
    }
    stash(0, 0, xl[0], al[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int k = kt + u;
        if (k >= nk) break;
        if constexpr (DEPTH == 1) {
          if (k + 1 < nk) issue(k + 1, xl[0], al[0]);
        } else {
          issue(k + DEPTH < nk ? k + DEPTH : nk - 1, xl[u], al[u]);
        }
        mma(k & 1, acc);
        if (k + 1 < nk) stash((k + 1) & 1, k + 1, xl[(u + 1) % DEPTH], al[(u + 1) % DEPTH]);
        __syncthreads();
      }
    }

    if (PAIR && p.ksplit > 1) {
      // Split K: this range's f32 partial (rows past the rank as zero),
      // written through to the device's coherence point, indexed by sorted
      // position; then the arrival count and, unless the stacked call's
      // expand sums the partials itself, the last arriver's reduction.
      const __amdgpu_buffer_rsrc_t prsrc = buffer_rsrc(p.partial, p.partial_bytes);
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const int mm = xr0 + 16 * f + frow;
        if (mm >= mcount) continue;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int n = nb * BN + (ar0 - BM) + 16 * i + 4 * fgrp;
          if (n >= p.CR) continue;
          f32x4 v = acc[i][f];
          const int j0 = n % p.R;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j0 + e >= rho) v[e] = 0.f;
          const int64_t idx = (static_cast<int64_t>(split) * p.s + (m0 + mm)) * p.CR + n;
          store_coherent16(prsrc, static_cast<uint32_t>(idx * 4), v);
        }
      }
      if (p.partials_only) continue;
      // (lo / BM + seg + mb) is distinct for every tile of a CSR plan
      detail::finish_split_tile(p, (static_cast<int64_t>(lo / BM) + seg + mb) * p.nblocks + nb,
                                m0, mcount, nb * BN, BN, &last_flag);
      continue;
    }

    // Epilogue: lane holds rank rows n .. n+3 of token column m for each
    // fragment; rows past the rank are stored as zero.
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int mm = xr0 + 16 * f + frow;
      if (mm >= mcount) continue;
      const int r = p.perm[m0 + mm];
      if (r < 0 || r >= p.s) continue;
      uint16_t* hrow = p.h + static_cast<int64_t>(r) * p.ldh;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = nb * BN + (ar0 - BM) + 16 * i + 4 * fgrp;
        if (n >= p.CR) continue;
        const f32x4 v = acc[i][f];
        const int j0 = n % p.R;  // rank index of n (n .. n+3 lie in one slice: R % 8 == 0)
        uint2 o;
        o.x = (j0 < rho ? f32_to_bf16(v[0]) : 0u) | ((j0 + 1 < rho ? f32_to_bf16(v[1]) : 0u) << 16);
        o.y = (j0 + 2 < rho ? f32_to_bf16(v[2]) : 0u) | ((j0 + 3 < rho ? f32_to_bf16(v[3]) : 0u) << 16);
        *reinterpret_cast<uint2*>(hrow + n) = o;
      }
    }
  }
}

template <int BM, int BN, int WM, int DEPTH, bool PAIR = false>
hipError_t launch_g(const ShrinkParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((shrink_gemm_kernel<BM, BN, WM, DEPTH, PAIR>),
                     dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Tile shapes with a kernel: (BM, BN) in {64, 128} x {32, 64, 128}; waves
// split BN in two where BN allows, else all four split BM.  Two register
// sets of prefetch except for 128 x 128 (one set: two would spill).
hipError_t launch_shrink_gemm(const ShrinkParams& p, int bm, int bn, int64_t grid,
                              hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (bm * 1000 + bn) {
    case 256128: return launch_g<256, 128, 2, 1, true>(p, grid, stream);
    case 128128: return launch_g<128, 128, 2, 1>(p, grid, stream);
    case 128064: return launch_g<128, 64, 2, 2>(p, grid, stream);
    case 128032: return launch_g<128, 32, 4, 2>(p, grid, stream);
    case 64128: return launch_g<64, 128, 2, 2>(p, grid, stream);
    case 64064: return launch_g<64, 64, 2, 2>(p, grid, stream);
    case 64032: return launch_g<64, 32, 4, 2>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sgg
