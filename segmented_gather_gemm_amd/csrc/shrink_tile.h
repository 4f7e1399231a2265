// LoRA-A shrink work item (one tile of one segment) and its block mapping.
// The algorithm is described at the top of shrink.hip.
#pragma once

#include "sgg_device.h"
#include "sgg_kernels.h"

namespace sgg {
namespace detail {

constexpr int kFragsPerRound = 8;  // accumulator fragments reduced per LDS round
constexpr int kValuTokens = 4;     // tiles of at most this many tokens take the VALU form

// a . b over 4 bf16 pairs (two 32-bit words each), accumulated in f32
__device__ __forceinline__ float dot4_bf16(uint2 a, uint2 b, float acc) {
  acc = fmaf(bf16_to_f32(a.x & 0xffffu), bf16_to_f32(b.x & 0xffffu), acc);
  acc = fmaf(bf16_to_f32(a.x >> 16), bf16_to_f32(b.x >> 16), acc);
  acc = fmaf(bf16_to_f32(a.y & 0xffffu), bf16_to_f32(b.y & 0xffffu), acc);
  acc = fmaf(bf16_to_f32(a.y >> 16), bf16_to_f32(b.y >> 16), acc);
  return acc;
}

// Byte offset of 16-byte chunk c (0..7) of row r in a swizzled 128-byte-row tile.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }

template <int MF, int NF>
struct ShrinkShape {
  static constexpr int BM = 16 * MF;
  static constexpr int NB = 16 * NF;
  static constexpr int NFR = MF * NF;
  static constexpr int ROWS = BM + NB;          // tile rows per chunk: x rows, then A rows
  static constexpr int LOADS = ROWS / 8;        // coalesced 16-byte loads per lane per chunk
  static constexpr int XL = BM / 8;             // of which x rows
  static constexpr int CH = ROWS >= 128 ? 1 : 128 / ROWS;  // chunks fetched per round trip
  static constexpr int ROUNDS = (NFR + kFragsPerRound - 1) / kFragsPerRound;
  static constexpr int STAGE_BYTES = 4 * CH * ROWS * 128;
  static constexpr int RED_BYTES = 4 * kFragsPerRound * kWave * 16;
  static constexpr int SMEM = STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES;
};

// Work item of block b: false for the padding blocks of the grid.
__device__ __forceinline__ bool shrink_item_of(const ShrinkParams& p, int b, int* seg, int* item) {
  const int per = p.mblocks * p.nblocks * p.ksplit;
  segment_round_robin(b, per, seg, item);
  return *seg < p.num_segments;
}

// Split-K completion of one tile -- rows [m0, m0 + mcount) of the sorted
// order by columns [n0, n0 + nb_cols) of c*R -- whose f32 partial went out
// with device-coherent stores.  Every wave waits for its own stores, then the
// barrier and one counter RMW (see wave_stores_done); the last of the
// ksplit workgroups to arrive reads the partials with device-coherent loads,
// sums them in split order (the order in which the stacked call's expand sums
// them too), writes bf16 h and resets the counter.  Every thread calls it;
// `cidx` is the tile's counter (clamped to the region).
__device__ inline void finish_split_tile(const ShrinkParams& p, int64_t cidx, int m0, int mcount,
                                         int n0, int nb_cols, int* last_flag) {
  const int tid = threadIdx.x;
  wave_stores_done();
  __syncthreads();
  if (cidx >= p.counter_cap) cidx = p.counter_cap - 1;
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(p.counters + cidx, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    *last_flag = old == p.ksplit - 1;
  }
  __syncthreads();
  if (!*last_flag) return;
  const __amdgpu_buffer_rsrc_t prsrc = buffer_rsrc(p.partial, p.partial_bytes);
  const int items = mcount * (nb_cols / 4);
  for (int q = tid; q < items; q += 256) {
    const int mm = q / (nb_cols / 4);
    const int n = n0 + 4 * (q % (nb_cols / 4));
    if (n >= p.CR) continue;
    const int r = p.perm[m0 + mm];
    if (r < 0 || r >= p.s) continue;
    // four splits' loads in flight at a time
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < p.ksplit; sp0 += 4) {
      f32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sp = sp0 + u < p.ksplit ? sp0 + u : sp0;
        const int64_t idx = (static_cast<int64_t>(sp) * p.s + (m0 + mm)) * p.CR + n;
        w[u] = load_coherent16(prsrc, static_cast<uint32_t>(idx * 4));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (sp0 + u < p.ksplit) v += w[u];
    }
    uint2 o;
    o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(p.h + static_cast<int64_t>(r) * p.ldh + n) = o;
  }
  if (tid == 0) __hip_atomic_store(p.counters + cidx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tile `item` of segment `seg`; `smem` holds ShrinkShape<MF, NF>::SMEM bytes.
// Every early return is uniform over the workgroup.
//
// VALU (MF == 1 only): a tile with at most kValuTokens tokens computes its
// dot products on the vector ALU instead of the matrix cores -- from the same
// staged chunks, so it reads the same bytes.  Lane (q, kp) = (lane / 16,
// lane % 16) takes 4 of each 64-deep chunk's k (4*kp .. 4*kp+3) for the rank
// rows 16g + 4q + e of the tile and every token; at the end each row group
// of 16 lanes sums its k parts by butterfly exchanges, so lane (q, kp) holds
// token kp's sums for its rows: the layout an MFMA accumulator has, and the
// four waves' tiles are summed and written as in the MFMA form.
template <int MF, int NF, bool VALU = false>
__device__ __forceinline__ void shrink_tile(const ShrinkParams& p, int seg, int item, char* smem,
                                            int* last_flag_ptr) {
  static_assert(!VALU || (MF == 1 && NF <= 3), "VALU tiles: 16 tokens, at most 48 rank rows");
  using S = ShrinkShape<MF, NF>;
  constexpr int BM = S::BM;
  constexpr int NB = S::NB;
  constexpr int NFR = S::NFR;
  constexpr int ROWS = S::ROWS;
  constexpr int LOADS = S::LOADS;
  constexpr int XL = S::XL;
  constexpr int CH = S::CH;
  constexpr int ROUNDS = S::ROUNDS;
  int& last_flag = *last_flag_ptr;
  f32x4 (*red)[kFragsPerRound][kWave] = reinterpret_cast<f32x4 (*)[kFragsPerRound][kWave]>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  char* tile = smem + wave * CH * ROWS * 128;
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
  // A tile whose rank rows all lie past the slot's rank (padding) is handled
  // like a rank-0 slot: nothing is read, split 0 alone writes the zero rows
  // (the expand masks h columns past the rank, so no partials are needed).
  bool tile_live = false;
  {
    const int n0 = nb * NB, n1 = min(n0 + NB, p.CR);
    for (int k = n0 / p.R; k * p.R < n1 && !tile_live; ++k)
      tile_live = max(n0, k * p.R) - k * p.R < rho;
  }
  const bool dead = rho == 0 || !tile_live;
  if (dead && split != 0) return;  // split 0 alone writes the zero rows

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
      // in-bounds stand-in for an invalid row, zeroed at the fragment read
      xrow[i] = (r >= 0 && r < p.s) ? (p.xdiv > 1 ? r / p.xdiv : r) : 0;
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
    // VALU form: per-lane sums for token t, rank row 16g + 4q + e
    const bool valu = VALU && mcount <= kValuTokens;
    constexpr int VT = VALU ? kValuTokens : 1;
    constexpr int VG = VALU ? NF : 1;
    float vacc[VT][VG][4];
    bool vtok[VT];
    if constexpr (VALU) {
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        bool ok = t < mcount;
        if (ok) {
          const int r = p.perm[m0 + t];
          ok = r >= 0 && r < p.s;
        }
        vtok[t] = ok;
#pragma unroll
        for (int g = 0; g < VG; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) vacc[t][g][e] = 0.f;
      }
    }
    const int vq = lane >> 4, vkp = lane & 15;

    if (!dead && nchunks > 0) {
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
          if constexpr (VALU) {
            if (valu) {
              // 8 bytes of 16-byte chunk vkp / 2 of each row
              const int c = vkp >> 1, off = 8 * (vkp & 1);
              const bool kv = k0 + 8 * c < ke;
              uint2 xv[VT];
#pragma unroll
              for (int tt = 0; tt < VT; ++tt) {
                const uint2 v = *reinterpret_cast<const uint2*>(ct + swz(tt, c) + off);
                xv[tt] = (kv && vtok[tt]) ? v : make_uint2(0, 0);
              }
#pragma unroll
              for (int g = 0; g < VG; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int nl = 16 * g + 4 * vq + e;
                  const int n = nb * NB + nl;
                  const uint2 v = *reinterpret_cast<const uint2*>(ct + swz(BM + nl, c) + off);
                  const uint2 av = (kv && n < p.CR && (n % p.R) < rho) ? v : make_uint2(0, 0);
#pragma unroll
                  for (int tt = 0; tt < VT; ++tt) vacc[tt][g][e] = dot4_bf16(av, xv[tt], vacc[tt][g][e]);
                }
              continue;
            }
          }
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

    if constexpr (VALU) {
      if (valu) {
        // butterfly over the 16 k parts of each row group, then token vkp's
        // sums into the accumulator layout (tokens past kValuTokens: zero)
#pragma unroll
        for (int tt = 0; tt < VT; ++tt)
#pragma unroll
          for (int g = 0; g < VG; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v = vacc[tt][g][e];
              v += __shfl_xor(v, 1, 64);
              v += __shfl_xor(v, 2, 64);
              v += __shfl_xor(v, 4, 64);
              v += __shfl_xor(v, 8, 64);
              vacc[tt][g][e] = v;
            }
#pragma unroll
        for (int g = 0; g < VG; ++g) {
          f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int tt = 0; tt < VT; ++tt)
            if (vkp == tt) a = f32x4{vacc[tt][g][0], vacc[tt][g][1], vacc[tt][g][2], vacc[tt][g][3]};
          acc[g] = a;
        }
      }
    }

    // Sum the four waves' tiles through LDS, a few fragments per round, and
    // emit 4 consecutive outputs of one token per (fragment, lane) item.
    const bool direct = p.ksplit == 1 || dead;
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
          // written through to the device's coherence point (no dirty L2 lines)
          const int64_t idx = (static_cast<int64_t>(split) * p.s + (m0 + mm)) * p.CR + n;
          store_coherent16(buffer_rsrc(p.partial, p.partial_bytes),
                           static_cast<uint32_t>(idx * 4), v);
        }
      }
    }
    if (direct || p.partials_only) continue;

    // Split-K: publish this partial, count arrivals, the last one reduces.
    // (lo / BM + seg + mb) is distinct for every (segment, row block) of a
    // CSR plan, so every tile has its own counter.
    finish_split_tile(p, (static_cast<int64_t>(lo / BM) + seg + mb) * p.nblocks + nb, m0,
                      mcount, nb * NB, NB, &last_flag);
  }
}

}  // namespace detail
}  // namespace sgg
