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
// Work order: column tiles are dealt to the XCDs (expand_item_of): each XCD
// takes every eighth tile of every segment, segment after segment, so it
// needs only one eighth of an adapter's B columns and reuses them from its L2
// across the adapter's consecutive segments, and every XCD gets an equal share
// of every segment however the tokens fall on the adapters.  (Dealing whole
// segments to the XCDs, the alternative kept behind the "expand_deal_tiles"
// option, re-fetched B from HBM per segment: the prefill expand read 1.24x its
// algorithmic bytes against 1.02x now.)
//
// With split-K partials (HPART, the stacked call) h is staged from them: each
// (row, 8-column chunk) sums its splits in split order in registers and
// rounds to bf16, the shrink's own reduction order, so the stacked call gives
// the separate calls' bits.
#include "sgg_device.h"
#include "sgg_kernels.h"
#include "expand_tile.h"

namespace sgg {

namespace {

template <int P, int KS, bool HPART>
__global__ __launch_bounds__(256) void expand_kernel(ExpandParams p) {
  __shared__ __attribute__((aligned(16))) char smem[detail::ExpandShape<P, KS>::SMEM];
  int seg, tile;
  if (!detail::expand_item_of(p, blockIdx.x, &seg, &tile)) return;
  detail::expand_tile<P, KS, HPART>(p, seg, tile, smem);
}

template <int P, bool HPART>
hipError_t launch_ph(const ExpandParams& p, int ks, int64_t grid, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>(grid)), b(256);
  switch (ks) {
    case 1: hipLaunchKernelGGL((expand_kernel<P, 1, HPART>), g, b, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((expand_kernel<P, 2, HPART>), g, b, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((expand_kernel<P, 4, HPART>), g, b, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int P>
hipError_t launch_p(const ExpandParams& p, int ks, int64_t grid, hipStream_t stream) {
  return p.hpart ? launch_ph<P, true>(p, ks, grid, stream) : launch_ph<P, false>(p, ks, grid, stream);
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

// Position-major form, for plans of at most kEmbedPosSegments segments
// (decode batches): one wave per 64 consecutive (sorted position, j) pairs.
// Each lane requests its position's permutation entry and, at the same time,
// one segment start (lane i: seg_indptr[i]); a ballot per position of the
// wave's window then finds the segment holding it, so the token id and the
// segment's slot come one round trip later and the table value one after
// that -- three dependent loads where the segment-major form above needs
// four.  The value is requested for every j < R and kept only below the
// rank, so the rank's load runs beside it.
constexpr int kEmbedPosSegments = 63;

__global__ __launch_bounds__(64) void embedding_pos_kernel(EmbeddingParams p) {
  const int lane = threadIdx.x;
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int64_t q = q0 + lane;
  const int64_t pos = q / p.R;
  const int j = static_cast<int>(q - pos * p.R);
  const int nseg = p.num_segments;
  const int start = lane <= nseg ? p.seg_indptr[lane] : 0;
  const int r = pos < p.s ? p.perm[pos] : -1;
  // segment of this lane's position: the last segment starting at or before
  // it, if the position lies before that segment's end
  int seg = -1;
  const int64_t p_first = q0 / p.R, p_last = (q0 + 63) / p.R;
  for (int64_t k = p_first; k <= p_last; ++k) {
    const uint64_t m = __ballot(lane < nseg && start <= k);
    if (m == 0) continue;
    const int sk = 63 - __builtin_clzll(m);
    const int end = __builtin_amdgcn_readlane(start, sk + 1);
    if (pos == k && k < end) seg = sk;
  }
  if (seg < 0 || r < 0 || r >= p.s || pos >= p.s) return;
  const int slot = p.seg_slots[seg];
  const int64_t id = p.ids[r];
  const bool slot_ok = slot >= 0 && slot < p.L;
  uint16_t v = 0;
  int rho = 0;
  if (slot_ok) {
    rho = p.ranks[slot];
    if (id >= 0 && id < p.vocab) v = p.A[(static_cast<int64_t>(slot) * p.R + j) * p.V + id];
  }
  rho = rho < 0 ? 0 : (rho > p.R ? p.R : rho);
  p.out[static_cast<int64_t>(r) * p.ldo + j] = j < rho ? v : 0;
}

}  // namespace

hipError_t launch_embedding(const EmbeddingParams& p, hipStream_t stream) {
  const int64_t pos_grid = (p.s * p.R + 63) / 64;
  if (p.num_segments <= kEmbedPosSegments && pos_grid < (int64_t{1} << 31)) {
    const int64_t grid = pos_grid;
    if (grid <= 0 || p.num_segments <= 0) return hipSuccess;
    hipLaunchKernelGGL(embedding_pos_kernel, dim3(static_cast<unsigned>(grid)), dim3(64), 0,
                       stream, p);
    return hipGetLastError();
  }
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

constexpr int kCopyThreads = 1024;
constexpr int kCopyDepth = 8;  // 8-byte loads in flight per thread

// One workgroup copies the whole plan.  Each thread requests DEPTH 8-byte
// pieces before storing any, so THREADS * DEPTH * 8 bytes of plan cost one
// host-memory round trip.  Once every thread has stored its pieces the
// staging buffer has been read in full; thread 0 then writes `done_value` to
// `done` (host memory, system scope), if given, so the host can reuse the
// staging buffer without an event.
template <int THREADS, int DEPTH>
__device__ __forceinline__ void copy_plan_block(const int32_t* src, int32_t* dst, int64_t n,
                                                int32_t* done, int32_t done_value) {
  const int64_t n2 = n >> 1;
  const uint64_t* s2 = reinterpret_cast<const uint64_t*>(src);
  uint64_t* d2 = reinterpret_cast<uint64_t*>(dst);
  for (int64_t i0 = threadIdx.x; i0 < n2; i0 += static_cast<int64_t>(THREADS) * DEPTH) {
    uint64_t v[DEPTH];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * THREADS;
      v[u] = i < n2 ? __hip_atomic_load(s2 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0;
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * THREADS;
      if (i < n2) d2[i] = v[u];
    }
  }
  if ((n & 1) && threadIdx.x == 0)
    dst[n - 1] = __hip_atomic_load(src + n - 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (done != nullptr) {
    __syncthreads();  // every thread's loads have returned (their values are stored)
    if (threadIdx.x == 0)
      __hip_atomic_store(done, done_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

__global__ __launch_bounds__(kCopyThreads) void plan_copy_kernel(const int32_t* src, int32_t* dst,
                                                                 int64_t n, int32_t* done,
                                                                 int32_t done_value) {
  copy_plan_block<kCopyThreads, kCopyDepth>(src, dst, n, done, done_value);
}

// Plan copy and the decode-shaped embedding lookup in one launch.  Workgroup
// 0 copies the plan (16 KB per host-memory round trip: the plan of 256
// decode tokens takes one, of 3072 three; deeper unrolling spills scalar
// registers).  Each other
// workgroup takes 128 consecutive (token, j) pairs, the position-major
// embedding's spread over the CUs: the token's slot comes from the kernel
// arguments at the same time as its id from the device, then the table
// value and the slot's rank (also an argument) together -- two dependent
// round trips, and no read of the plan, which is still in flight.  As in
// the other forms, the value is requested for every j < R and kept only
// below the rank.
constexpr int kEmbedUploadThreads = 128;
constexpr int kEmbedUploadDepth = 16;

__global__ __launch_bounds__(kEmbedUploadThreads) void plan_copy_embedding_kernel(
    EmbedUploadParams p) {
  if (blockIdx.x == 0) {
    copy_plan_block<kEmbedUploadThreads, kEmbedUploadDepth>(p.src, p.dst, p.n, p.done,
                                                            p.done_value);
    return;
  }
  const int q = static_cast<int>(blockIdx.x - 1) * kEmbedUploadThreads + threadIdx.x;
  const int t = q / p.R;
  if (t >= p.s) return;
  const int j = q - t * p.R;
  const int slot = p.slot[t];
  const int64_t id = p.ids[t];
  const int rho = p.rank[slot];
  uint16_t v = 0;
  if (id >= 0 && id < p.vocab) v = p.A[(static_cast<int64_t>(slot) * p.R + j) * p.V + id];
  p.out[static_cast<int64_t>(t) * p.ldo + j] = j < rho ? v : 0;
}

}  // namespace

hipError_t launch_plan_copy(const int32_t* src_dev_view, int32_t* dst, int64_t n,
                            int32_t* done_dev_view, int32_t done_value, hipStream_t stream) {
  if (n <= 0 && done_dev_view == nullptr) return hipSuccess;
  hipLaunchKernelGGL(plan_copy_kernel, dim3(1), dim3(kCopyThreads), 0, stream, src_dev_view, dst,
                     n < 0 ? 0 : n, done_dev_view, done_value);
  return hipGetLastError();
}

hipError_t launch_plan_copy_embedding(const EmbedUploadParams& p, hipStream_t stream) {
  const int64_t pairs = static_cast<int64_t>(p.s) * p.R;
  const int64_t grid = 1 + (pairs + kEmbedUploadThreads - 1) / kEmbedUploadThreads;
  hipLaunchKernelGGL(plan_copy_embedding_kernel, dim3(static_cast<unsigned>(grid)),
                     dim3(kEmbedUploadThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sgg
