// LoRA-A shrink: h[t, k*R + j] = sum_q A[a(t), k*R + j, q] * x[t, q] over the
// segments of a chunked plan (chunked_backend.py page: run_lora_a_sgemm and
// the shrink step of run_qkv_lora / run_gate_up_lora).
//
// One workgroup (4 waves) owns a tile of up to 16*MF tokens of one segment
// (gathered through the permutation) by 16*NF outputs of the c*R stacked
// rank rows, over one range of K.  The four waves walk interleaved 32-deep
// K steps of that range, each keeping the whole tile in its own MFMA
// accumulators, so no operand is loaded twice and the main loop needs no
// barrier; the four partial tiles are summed once through LDS at the end.
// Both operands are K-contiguous in memory (x rows and A rows), so each lane
// fetches its MFMA fragment as one 16-byte load straight from global memory.
//
// When the segments alone cannot fill the GPU (decode batches) K is also
// split across workgroups: each writes an f32 partial tile and bumps an
// arrival counter; the last to arrive sums the partials in split order
// (deterministic) and writes bf16 h, then resets the counter.
#include "sgg_device.h"
#include "sgg_internal.h"
#include "sgg_kernels.h"

namespace sgg {

namespace {

constexpr int kFragsPerRound = 8;  // accumulator fragments reduced per LDS round

template <int MF, int NF>
__global__ __launch_bounds__(256, 1) void shrink_kernel(ShrinkParams p) {
  constexpr int BM = 16 * MF;
  constexpr int NB = 16 * NF;
  constexpr int NFR = MF * NF;
  constexpr int ROUNDS = (NFR + kFragsPerRound - 1) / kFragsPerRound;
  __shared__ f32x4 red[4][kFragsPerRound][kWave];
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int L = xcd_contiguous(blockIdx.x, gridDim.x);
  const int mb0 = L % p.mblocks;
  L /= p.mblocks;
  const int seg = L % p.num_segments;
  L /= p.num_segments;
  const int nb = L % p.nblocks;
  const int split = L / p.nblocks;

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
  const int koff = 8 * (lane >> 4);

  // Weight rows held by this lane (same for every row block).
  const uint16_t* arow[NF];
  bool nvalid[NF];
#pragma unroll
  for (int g = 0; g < NF; ++g) {
    const int n = nb * NB + 16 * g + (lane & 15);
    nvalid[g] = n < p.CR && (n % p.R) < rho;
    arow[g] = p.A + (static_cast<int64_t>(a) * p.CR + (nvalid[g] ? n : 0)) * p.K;
  }

  for (int mb = mb0; lo + mb * BM < hi; mb += p.mblocks) {
    const int m0 = lo + mb * BM;
    const int mcount = hi - m0 < BM ? hi - m0 : BM;
    const int mf_act = (mcount + 15) >> 4;

    const uint16_t* xrow[MF];
    bool tvalid[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      const int mm = 16 * f + (lane & 15);
      tvalid[f] = false;
      xrow[f] = p.x;
      if (mm < mcount) {
        const int r = p.perm[m0 + mm];
        if (r >= 0 && r < p.s) {
          tvalid[f] = true;
          xrow[f] = p.x + static_cast<int64_t>(r) * p.ldx;
        }
      }
    }

    f32x4 acc[NFR];
#pragma unroll
    for (int i = 0; i < NFR; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (rho > 0) {
      // Two 32-deep steps per trip: all fragment loads of both are issued
      // before the first MFMA so their latencies overlap.
      for (int64_t k0 = kb + 32 * wave; k0 < ke; k0 += 256) {
        const int64_t k1 = k0 + koff;
        const int64_t k2 = k1 + 128;
        const bool kv1 = k1 < ke, kv2 = k2 < ke;
        uint4 xv1[MF], xv2[MF], av1[NF], av2[NF];
#pragma unroll
        for (int f = 0; f < MF; ++f) {
          xv1[f] = make_uint4(0, 0, 0, 0);
          xv2[f] = make_uint4(0, 0, 0, 0);
          if (f < mf_act && tvalid[f]) {
            if (kv1) xv1[f] = load16(xrow[f] + k1);
            if (kv2) xv2[f] = load16(xrow[f] + k2);
          }
        }
#pragma unroll
        for (int g = 0; g < NF; ++g) {
          av1[g] = make_uint4(0, 0, 0, 0);
          av2[g] = make_uint4(0, 0, 0, 0);
          if (nvalid[g]) {
            if (kv1) av1[g] = load16(arow[g] + k1);
            if (kv2) av2[g] = load16(arow[g] + k2);
          }
        }
#pragma unroll
        for (int f = 0; f < MF; ++f) {
          if (f < mf_act) {
#pragma unroll
            for (int g = 0; g < NF; ++g) acc[f * NF + g] = mfma16x16x32(av1[g], xv1[f], acc[f * NF + g]);
          }
        }
        if (k0 + 128 < ke) {
#pragma unroll
          for (int f = 0; f < MF; ++f) {
            if (f < mf_act) {
#pragma unroll
              for (int g = 0; g < NF; ++g) acc[f * NF + g] = mfma16x16x32(av2[g], xv2[f], acc[f * NF + g]);
            }
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
          float* dst = p.partial + (static_cast<int64_t>(split) * p.s + (m0 + mm)) * p.CR + n;
          *reinterpret_cast<f32x4*>(dst) = v;
        }
      }
    }
    if (direct) continue;

    // Split-K: publish this partial, count arrivals, the last one reduces.
    __threadfence();
    __syncthreads();
    // (lo / BM + seg + mb) is distinct for every (segment, row block) of a
    // CSR plan, so every tile has its own counter; the clamp only keeps a
    // malformed plan in bounds.
    int64_t cidx = (static_cast<int64_t>(lo / BM) + seg + mb) * p.nblocks + nb;
    if (cidx >= p.counter_cap) cidx = p.counter_cap - 1;
    if (tid == 0) {
      const int old = atomicAdd(p.counters + cidx, 1);
      last_flag = (old == p.ksplit - 1);
    }
    __syncthreads();
    if (!last_flag) continue;
    __threadfence();
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
        v += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
      }
      uint2 o;
      o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(p.h + static_cast<int64_t>(r) * p.ldh + n) = o;
    }
    if (tid == 0) atomicExch(p.counters + cidx, 0);
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

// Fragment counts: NF covers c*R (at most 8 fragments = 128 outputs per
// column block), MF the chunk (at most 8 fragments = 128 tokens), with at
// most 32 accumulator fragments per wave.  K is split across workgroups only
// when segments x column blocks cannot give every CU a workgroup.
ShrinkTiling choose_shrink_tiling(int64_t s, int64_t K, int CR, int num_segments, int chunk) {
  ShrinkTiling t{};
  const int need = (CR + 15) / 16;
  static const int kNf[] = {1, 2, 3, 4, 6, 8};
  t.nf = 8;
  for (int v : kNf) {
    if (v >= need) {
      t.nf = v;
      break;
    }
  }
  t.nblocks = (CR + 16 * t.nf - 1) / (16 * t.nf);
  const int chunk16 = (chunk < 16 ? 16 : chunk + 15) / 16;
  t.mf = 1;
  for (int v : {8, 4, 2, 1}) {
    if (v * t.nf <= 32 && v <= chunk16) {
      t.mf = v;
      break;
    }
  }
  const int bm = 16 * t.mf;
  t.mblocks = (chunk + bm - 1) / bm;
  if (t.mblocks < 1) t.mblocks = 1;
  const int64_t units_grid = static_cast<int64_t>(num_segments) * t.mblocks;
  const int64_t units_real = (s + bm - 1) / bm + num_segments;
  const int64_t units = (units_grid < units_real ? units_grid : units_real) * t.nblocks;
  const int64_t kgroups = (K + 127) / 128;
  int64_t ksplit = 1;
  const int64_t counters = (s / bm + num_segments + 1) * t.nblocks;
  if (units > 0 && units < 256 && counters <= kCounterCap) {
    ksplit = (256 + units - 1) / units;
    if (ksplit > kgroups) ksplit = kgroups;
  }
  t.kps = (kgroups + ksplit - 1) / ksplit * 128;
  t.ksplit = static_cast<int>((K + t.kps - 1) / t.kps);
  if (t.ksplit < 1) t.ksplit = 1;
  t.grid = static_cast<int64_t>(t.ksplit) * t.nblocks * num_segments * t.mblocks;
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
