// LoRA-B expand: out[t, o_k + n] += sigma_a * sum_{j<rho_a} B[a, o_k + n, j] *
// h[t, k*R + j] over the segments of a chunked plan (chunked_backend.py page:
// run_lora_b_sgemm and the expand step of run_qkv_lora / run_gate_up_lora).
//
// One workgroup (4 waves) owns one segment and one tile of 64*NFW columns of
// one slice.  Each wave loads the B fragments of its 16*NFW columns into
// registers once (the rank is the short contraction dimension) and then walks
// the segment 16 tokens at a time: one 16-byte h fragment per lane, KS MFMAs
// per 16 columns, and a read-modify-write of the base rows.  The MFMA is set
// up as out^T = B * h^T so that each lane ends with 4 consecutive columns of
// one token: the base update is an 8-byte access per lane.
#include "sgg_device.h"
#include "sgg_kernels.h"

namespace sgg {

namespace {

template <int NFW, int KS>
__global__ __launch_bounds__(256) void expand_kernel(ExpandParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int L = xcd_contiguous(blockIdx.x, gridDim.x);
  const int seg = L % p.num_segments;
  const int tile = L / p.num_segments;

  int k = 0;
  while (k + 1 < p.c && tile >= p.tile_start[k + 1]) ++k;
  const int col0 = p.offs[k] + (tile - p.tile_start[k]) * (64 * NFW) + 16 * NFW * wave;
  const int colend = p.offs[k + 1];
  if (col0 >= colend) return;

  // segment bounds, clamped to [0, s) so a malformed plan stays in bounds
  const int lo = max(p.seg_indptr[seg], 0);
  const int hi = min(static_cast<int64_t>(p.seg_indptr[seg + 1]), p.s);
  if (hi <= lo) return;
  const int slot = p.seg_slots[seg];
  int rho = (slot >= 0 && slot < p.L) ? p.ranks[slot] : 0;
  rho = rho < 0 ? 0 : (rho > p.R ? p.R : rho);
  if (rho == 0) return;  // base model: output rows stay untouched
  const float sigma = p.scalings[slot];
  const int j8 = 8 * (lane >> 4);

  // B fragments: rows n of slice k, rank columns j8 + 32*ks .. +7.
  uint4 bw[NFW][KS];
#pragma unroll
  for (int g = 0; g < NFW; ++g) {
    const int n = col0 + 16 * g + (lane & 15);
    const uint16_t* brow = p.B + (static_cast<int64_t>(slot) * p.N + n) * p.R;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int j = 32 * ks + j8;
      bw[g][ks] = make_uint4(0, 0, 0, 0);
      if (n < colend && j < rho) bw[g][ks] = keep_first(load16(brow + j), rho - j);
    }
  }

  const int hcol = k * p.R;
  for (int m0 = lo; m0 < hi; m0 += 16) {
    const int tok = m0 + (lane & 15);
    int row = -1;
    if (tok < hi) {
      const int r = p.perm[tok];
      if (r >= 0 && r < p.s) row = r;
    }
    uint4 hv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int j = 32 * ks + j8;
      hv[ks] = make_uint4(0, 0, 0, 0);
      if (row >= 0 && j < rho)
        hv[ks] = keep_first(load16(p.h + static_cast<int64_t>(row) * p.ldh + hcol + j), rho - j);
    }
    uint16_t* orow = p.out + static_cast<int64_t>(row < 0 ? 0 : row) * p.ldo;
    // Base values first, so their latency overlaps the MFMAs.
    uint2 bv[NFW];
#pragma unroll
    for (int g = 0; g < NFW; ++g) {
      const int c4 = col0 + 16 * g + 4 * (lane >> 4);
      bv[g] = make_uint2(0, 0);
      if (row >= 0 && p.vec4 && c4 + 4 <= colend)
        bv[g] = *reinterpret_cast<const uint2*>(orow + c4);
    }
#pragma unroll
    for (int g = 0; g < NFW; ++g) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(bw[g][ks], hv[ks], acc);
      const int c4 = col0 + 16 * g + 4 * (lane >> 4);
      if (row < 0 || c4 >= colend) continue;
      if (p.vec4 && c4 + 4 <= colend) {
        const float y0 = bf16_to_f32(bv[g].x & 0xffffu) + sigma * acc[0];
        const float y1 = bf16_to_f32(bv[g].x >> 16) + sigma * acc[1];
        const float y2 = bf16_to_f32(bv[g].y & 0xffffu) + sigma * acc[2];
        const float y3 = bf16_to_f32(bv[g].y >> 16) + sigma * acc[3];
        uint2 o;
        o.x = f32_to_bf16(y0) | (f32_to_bf16(y1) << 16);
        o.y = f32_to_bf16(y2) | (f32_to_bf16(y3) << 16);
        *reinterpret_cast<uint2*>(orow + c4) = o;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (c4 + i < colend) {
            const float y = bf16_to_f32(orow[c4 + i]) + sigma * acc[i];
            orow[c4 + i] = static_cast<uint16_t>(f32_to_bf16(y));
          }
        }
      }
    }
  }
}

template <int NFW>
hipError_t launch_w(const ExpandParams& p, int ks, int64_t grid, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>(grid)), b(256);
  switch (ks) {
    case 1: hipLaunchKernelGGL((expand_kernel<NFW, 1>), g, b, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((expand_kernel<NFW, 2>), g, b, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((expand_kernel<NFW, 4>), g, b, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expand(const ExpandParams& p, const ExpandTiling& t, hipStream_t stream) {
  if (t.grid <= 0) return hipSuccess;
  switch (t.nfw) {
    case 1: return launch_w<1>(p, t.ks, t.grid, stream);
    case 2: return launch_w<2>(p, t.ks, t.grid, stream);
    case 4: return launch_w<4>(p, t.ks, t.grid, stream);
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

}  // namespace sgg
