// LoRA-B expand: out[t, o_k + n] += sigma_a * sum_{j<rho_a} B[a, o_k + n, j] *
// h[t, k*R + j] over the segments of a chunked plan (chunked_backend.py page:
// run_lora_b_sgemm and the expand step of run_qkv_lora / run_gate_up_lora).
//
// One workgroup (4 waves) owns one segment and one tile of 128*P columns of
// one slice; each wave owns 32*P of those columns and keeps their B rows in
// registers as MFMA fragments (the rank is the short contraction dimension).
// The segment is walked 128 tokens at a time: the h rows of those tokens
// (slice k's R columns) are fetched once per workgroup, coalesced, into a
// swizzled LDS tile that all waves read their fragments from.  Then, 16
// tokens at a time, each wave computes out^T = B * h^T on the MFMA and
// transposes the accumulators through a padded LDS tile so that the base
// rows are read and written coalesced: 4*P lanes cover the 64*P contiguous
// bytes of one row.  The base rows of the next 16 tokens are in flight while
// the current ones are computed and stored.
//
// Work order: each XCD takes a contiguous range of (segment, tile) items with
// tiles fastest, so the workgroups resident on an XCD sweep whole rows of the
// base tensor and share the segment's h rows and its adapter's B tiles in L2.
// With few segments (e.g. a capacity-padded graph launch, whose trailing
// segments are empty) segments are dealt round-robin to the XCDs instead.
#include "sgg_device.h"
#include "sgg_kernels.h"

namespace sgg {

namespace {

template <int P, int KS>
__global__ __launch_bounds__(256) void expand_kernel(ExpandParams p) {
  constexpr int TNW = 32 * P;                  // columns per wave
  constexpr int CPR = 4 * KS;                  // 16-byte chunks per LDS h row (R <= 32*KS)
  constexpr int RPS = 16 / CPR > 0 ? 16 / CPR : 1;  // h rows sharing one swizzle value
  constexpr int LPR = 4 * P;                   // lanes per base row segment (16 B each)
  constexpr int RPL = 64 / LPR;                // base rows per wave load
  constexpr int BLD = 16 / RPL;                // base loads per 16 tokens
  constexpr int APAD = TNW + 4;                // floats per row of the transpose tile
  __shared__ uint4 htile[128 * CPR];
  __shared__ int prow[128];
  __shared__ __attribute__((aligned(16))) float acct[4][16 * APAD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int seg, tile;
  if (p.round_robin) {
    segment_round_robin(blockIdx.x, p.total_tiles, &seg, &tile);
    if (seg >= p.num_segments) return;
  } else {
    const int L = xcd_contiguous(blockIdx.x, gridDim.x);
    seg = L / p.total_tiles;
    tile = L % p.total_tiles;
  }

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
  // Requested before the slot's rank arrives (every column j < R is in
  // bounds); columns at or beyond the rank are zeroed once it is known.
  uint4 bw[2 * P][KS];
#pragma unroll
  for (int g = 0; g < 2 * P; ++g) {
    const int n = colw + 16 * g + m;
    const uint16_t* brow =
        p.B + (static_cast<int64_t>(slot_ok ? slot : 0) * p.N + (n < colend ? n : 0)) * p.R;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int j = 32 * ks + 8 * q;
      bw[g][ks] = make_uint4(0, 0, 0, 0);
      if (active && n < colend && j < p.R) bw[g][ks] = load16(brow + j);
    }
  }
  int rho = slot_ok ? p.ranks[slot] : 0;
  rho = rho < 0 ? 0 : (rho > p.R ? p.R : rho);
  if (rho == 0) return;  // base model: output rows stay untouched
  const float sigma = p.scalings[slot];
#pragma unroll
  for (int g = 0; g < 2 * P; ++g)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bw[g][ks] = keep_first(bw[g][ks], rho - (32 * ks + 8 * q));

  // Base-row role of this lane: row (RPL*i + lane/LPR) of a 16-token group,
  // columns colw + 8*(lane%LPR) .. +7.
  const int brw = lane / LPR;
  const int bc = colw + 8 * (lane % LPR);
  const bool bvec = p.vec8 && bc + 8 <= colend;
  const int hch = p.R >> 3;  // 16-byte chunks of one h row slice
  float* at = acct[wave];

  for (int c0 = lo; c0 < hi; c0 += 128) {
    const int ntok = hi - c0 < 128 ? hi - c0 : 128;
    __syncthreads();  // previous chunk's tiles are no longer read
    if (tid < ntok) {
      const int r = p.perm[c0 + tid];
      prow[tid] = (r >= 0 && r < p.s) ? r : -1;
    }
    if (p.hpart) {
      // split-K partials, indexed by sorted position: no gather needed
      for (int piece = tid; piece < ntok * hch; piece += 256) {
        const int row = piece / hch, c = piece % hch;
        const float* src = p.hpart + static_cast<int64_t>(c0 + row) * p.ldp + k * p.R + 8 * c;
        f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
        for (int sp = 0; sp < p.hsplit; ++sp) {
          const float* q = src + static_cast<int64_t>(sp) * p.s * p.ldp;
          s0 += *reinterpret_cast<const f32x4*>(q);
          s1 += *reinterpret_cast<const f32x4*>(q + 4);
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
    fetch(0, bv0);
    for (int f = 0; f < nf; f += 2) {
      if (f + 1 < nf) fetch(f + 1, bv1);
      step(f, bv0);
      if (f + 1 < nf) {
        if (f + 2 < nf) fetch(f + 2, bv0);
        step(f + 1, bv1);
      }
    }
  }
}

template <int P>
hipError_t launch_p(const ExpandParams& p, int ks, int64_t grid, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>(grid)), b(256);
  switch (ks) {
    case 1: hipLaunchKernelGGL((expand_kernel<P, 1>), g, b, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((expand_kernel<P, 2>), g, b, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((expand_kernel<P, 4>), g, b, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expand(const ExpandParams& p, const ExpandTiling& t, hipStream_t stream) {
  if (t.grid <= 0) return hipSuccess;
  switch (t.pairs) {
    case 1: return launch_p<1>(p, t.ks, t.grid, stream);
    case 2: return launch_p<2>(p, t.ks, t.grid, stream);
    case 4: return launch_p<4>(p, t.ks, t.grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------- embedding
// LoRA-A embedding lookup (chunked_backend.py page: run_lora_a_embedding):
// out[t, j] = A_emb[a(t), j, ids[t]] for j < rho_a, in-vocabulary ids.
// Workgroup (segment, part) covers a strided share of the segment's
// (token, j) pairs; consecutive threads take consecutive j of one token, so
// the output row is written contiguously.  The reads are one column of A_emb
// (stride V) per token: latency-bound, so each thread keeps several in flight.

namespace {

__global__ __launch_bounds__(256) void embedding_kernel(EmbeddingParams p) {
  const int seg = blockIdx.x % p.num_segments;
  const int part = blockIdx.x / p.num_segments;
  // segment bounds, clamped to [0, s) so a malformed plan stays in bounds
  const int lo = max(p.seg_indptr[seg], 0);
  const int hi = min(static_cast<int64_t>(p.seg_indptr[seg + 1]), p.s);
  if (hi <= lo) return;
  const int slot = p.seg_slots[seg];
  int rho = (slot >= 0 && slot < p.L) ? p.ranks[slot] : 0;
  rho = rho < 0 ? 0 : (rho > p.R ? p.R : rho);
  const int64_t pairs = static_cast<int64_t>(hi - lo) * p.R;
  const int64_t stride = static_cast<int64_t>(p.parts) * 256;
  constexpr int U = 4;
  for (int64_t q0 = static_cast<int64_t>(part) * 256 + threadIdx.x; q0 < pairs; q0 += U * stride) {
    int rows[U];
    int js[U];
    uint16_t vals[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = q0 + u * stride;
      rows[u] = -1;
      js[u] = 0;
      if (q < pairs) {
        const int r = p.perm[lo + static_cast<int>(q / p.R)];
        if (r >= 0 && r < p.s) rows[u] = r;
        js[u] = static_cast<int>(q % p.R);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vals[u] = 0;
      if (rows[u] >= 0 && js[u] < rho) {
        const int64_t id = p.ids[rows[u]];
        if (id >= 0 && id < p.vocab)
          vals[u] = p.A[(static_cast<int64_t>(slot) * p.R + js[u]) * p.V + id];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (rows[u] >= 0) p.out[static_cast<int64_t>(rows[u]) * p.ldo + js[u]] = vals[u];
  }
}

}  // namespace

hipError_t launch_embedding(const EmbeddingParams& p, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(p.num_segments) * p.parts;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(embedding_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// ------------------------------------------------------------- plan upload
// Copies the plan from pinned host memory to the device plan buffer.  A plain
// kernel on the caller's stream (system-scope loads, so each read sees the
// host's latest writes): small host-to-device copies through the runtime
// were seen to busy-wait on the host for the stream to drain.

namespace {

// Each thread issues its four loads before any store, so a small plan costs
// one host-memory round trip rather than one per element.
__global__ __launch_bounds__(256) void plan_copy_kernel(const int32_t* src, int32_t* dst, int64_t n) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i0 < n; i0 += 4 * step) {
    int32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * step;
      v[u] = i < n ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * step;
      if (i < n) dst[i] = v[u];
    }
  }
}

}  // namespace

hipError_t launch_plan_copy(const int32_t* src_dev_view, int32_t* dst, int64_t n,
                            hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 1023) / 1024;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(plan_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     src_dev_view, dst, n);
  return hipGetLastError();
}

}  // namespace sgg
