// The batch plan computed on the GPU (chunked_backend.py page:
// _determine_chunk_size, _get_permutation, _get_segments_info and
// _build_req_seg_indptr, with the CUDA-graph branch of prepare_lora_batch
// padding the segment arrays to a fixed capacity).  The same plan as the
// host planner, bit for bit, written straight into the device plan buffer
// from request lengths and slots that are already in device memory: no
// host round trip, and the launch can be captured in a graph together with
// the kernels that read the plan.
//
// One workgroup of 1024 threads:
//   1. request boundaries (a block-wide scan of the lengths), validation;
//   2. tokens per slot (LDS histogram), the chunk size, each slot's first
//      sorted position and first segment (scans over the slots);
//   3. each request's first sorted position: the stable counting sort.  One
//      wave walks the requests 64 at a time; a lane adds the lengths of
//      earlier lanes of its slot and the slot's running total, and the
//      slot's first lane in the group then advances that total;
//   4. the permutation: every thread takes tokens, finds each token's
//      request by binary search and writes its sorted position;
//   5. segments (full chunks, remainder last), work segments (consecutive
//      segments of one slot merged greedily within max(chunk, 128) tokens),
//      capacity padding (slot 0, zero length) and the rank / scaling tables.
// An invalid batch (a slot outside [0, L), a negative length, a decode
// request of other than one token, more tokens or segments than the
// capacities) is not planned: the status goes to info[6] and every segment
// and work segment is written empty, so the kernels that follow do nothing.
#include "sgg_device.h"
#include "sgg_internal.h"
#include "sgg_kernels.h"
#include "../../include/sgg_lora.h"

namespace sgg {

namespace {

constexpr int kPlanThreads = 1024;

struct DevicePlanParams {
  const int32_t* seq_lens;  // [bs], or null: one token per request (decode)
  const int32_t* req_slots;
  const int32_t* ranks;
  const float* scalings;
  int32_t* plan;            // device plan buffer (regions 0-8 of the layout)
  int32_t* info;            // [8]: n_seg, chunk, longest, tokens, n_work, longest work, status
  int64_t off[SGG_PLAN_REGIONS];
  int64_t token_capacity;
  int32_t bs, L, is_decode, max_chunk, chunk_override, seg_capacity;
};

__device__ __forceinline__ int chunk_for(int64_t n, int max_chunk) {
  if (max_chunk <= SGG_MIN_CHUNK_SIZE) return SGG_MIN_CHUNK_SIZE;
  const int wanted = n >= 256 ? 128 : (n >= 64 ? 32 : 16);
  return wanted < max_chunk ? wanted : max_chunk;
}

// Exclusive scan of v over the workgroup; returns the prefix and writes the
// total to *total.  Every thread must call it.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* wave_sums, int64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_sums[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t acc = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      const int64_t t = wave_sums[w];
      wave_sums[w] = acc;
      acc += t;
    }
    wave_sums[kPlanThreads / 64] = acc;
  }
  __syncthreads();
  const int64_t prefix = wave_sums[wave] + x - v;
  *total = wave_sums[kPlanThreads / 64];
  __syncthreads();
  return prefix;
}

__global__ __launch_bounds__(kPlanThreads) void plan_device_kernel(DevicePlanParams p) {
  __shared__ int32_t count[kDevicePlanMaxLoras];      // tokens per slot
  __shared__ int32_t first_pos[kDevicePlanMaxLoras];  // first sorted position per slot
  __shared__ int32_t running[kDevicePlanMaxLoras];    // next sorted position per slot
  __shared__ int32_t first_seg[kDevicePlanMaxLoras];  // first segment per slot
  __shared__ int32_t first_work[kDevicePlanMaxLoras]; // first work segment per slot
  __shared__ int32_t req_ptr[kDevicePlanMaxReqs + 1]; // request token boundaries
  __shared__ int32_t req_pos[kDevicePlanMaxReqs];     // first sorted position per request
  __shared__ int64_t wave_sums[kPlanThreads / 64 + 1];
  __shared__ int32_t status, longest, longest_work;

  const int tid = threadIdx.x;
  const int bs = p.bs, L = p.L;
  int32_t* perm = p.plan + p.off[0];
  int32_t* seg_indptr = p.plan + p.off[1];
  int32_t* seg_slots = p.plan + p.off[2];
  int32_t* req_indptr = p.plan + p.off[3];
  int32_t* req_slots_out = p.plan + p.off[4];
  int32_t* ranks_out = p.plan + p.off[5];
  int32_t* scal_out = p.plan + p.off[6];
  int32_t* work_indptr = p.plan + p.off[7];
  int32_t* work_slots = p.plan + p.off[8];

  if (tid == 0) {
    status = SGG_OK;
    longest = 0;
    longest_work = 0;
  }
  if (tid < L) count[tid] = 0;
  __syncthreads();

  // 1. Request boundaries and validation; tokens per slot.
  int64_t carry = 0;
  for (int r0 = 0; r0 < bs; r0 += kPlanThreads) {
    const int r = r0 + tid;
    int len = 0;
    if (r < bs) {
      len = p.seq_lens ? p.seq_lens[r] : 1;
      const int a = p.req_slots[r];
      if (len < 0 || (p.is_decode && len != 1)) atomicOr(&status, 1);
      if (a < 0 || a >= L) atomicOr(&status, 2);
      else if (len > 0) atomicAdd(&count[a], len);
      req_slots_out[r] = a;
    }
    int64_t chunk_total;
    const int64_t pre = block_exclusive_scan(len > 0 ? len : 0, wave_sums, &chunk_total);
    if (r < bs) {
      const int64_t end = carry + pre + (len > 0 ? len : 0);
      if (end > INT32_MAX) atomicOr(&status, 4);
      req_ptr[r + 1] = static_cast<int32_t>(end);
      req_indptr[r + 1] = static_cast<int32_t>(end);
    }
    carry += chunk_total;
  }
  if (tid == 0) {
    req_ptr[0] = 0;
    req_indptr[0] = 0;
  }
  const int64_t s = carry;
  if (s > p.token_capacity) {
    if (tid == 0) atomicOr(&status, 4);
  }
  __syncthreads();

  // 2. Chunk size; each slot's first sorted position, first segment and
  // first work segment (one slot per thread: L <= kPlanThreads).
  const int chunk = p.chunk_override > 0 ? p.chunk_override
                                         : chunk_for(p.is_decode ? bs : s, p.max_chunk);
  const int cap = chunk > SGG_WORK_SEGMENT_TOKENS ? chunk : SGG_WORK_SEGMENT_TOKENS;
  const int n_slot = tid < L ? count[tid] : 0;
  const int segs = (n_slot + chunk - 1) / chunk;
  int works = 0;  // work segments: the slot's segments merged greedily within `cap`
  for (int q = 0; q < segs;) {
    int tok = 0, q1 = q;
    while (q1 < segs) {
      const int len = q1 < segs - 1 ? chunk : n_slot - (segs - 1) * chunk;
      if (q1 > q && tok + len > cap) break;
      tok += len;
      ++q1;
    }
    ++works;
    q = q1;
  }
  int64_t tot_tok, n_seg, n_work;
  const int64_t pos = block_exclusive_scan(n_slot, wave_sums, &tot_tok);
  const int64_t sg = block_exclusive_scan(segs, wave_sums, &n_seg);
  const int64_t wk = block_exclusive_scan(works, wave_sums, &n_work);
  if (tid < L) {
    first_pos[tid] = static_cast<int32_t>(pos);
    first_seg[tid] = static_cast<int32_t>(sg);
    first_work[tid] = static_cast<int32_t>(wk);
  }
  if (tid == 0 && n_seg > p.seg_capacity) atomicOr(&status, 8);
  __syncthreads();
  const int st = status;

  if (st != SGG_OK) {
    // not planned: every segment and work segment empty
    for (int i = tid; i <= p.seg_capacity; i += kPlanThreads) {
      seg_indptr[i] = 0;
      work_indptr[i] = 0;
      if (i < p.seg_capacity) {
        seg_slots[i] = 0;
        work_slots[i] = 0;
      }
    }
    if (tid == 0) {
      p.info[0] = 0;
      p.info[1] = chunk;
      p.info[2] = 0;
      p.info[3] = 0;
      p.info[4] = 0;
      p.info[5] = 0;
      p.info[6] = st;
    }
    return;
  }

  // 3. First sorted position of each request (stable counting sort).
  for (int a = tid; a < L; a += kPlanThreads) running[a] = first_pos[a];
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    for (int r0 = 0; r0 < bs; r0 += 64) {
      const int r = r0 + lane;
      const int a = r < bs ? p.req_slots[r] : -1;
      const int len = r < bs ? req_ptr[r + 1] - req_ptr[r] : 0;
      int before = 0, group = 0;
      bool first = true;
      for (int j = 0; j < 64; ++j) {
        const int aj = __shfl(a, j, 64);
        const int lj = __shfl(len, j, 64);
        if (aj == a) {
          group += lj;
          if (j < lane) {
            before += lj;
            first = false;
          }
        }
      }
      const int base = r < bs ? running[a] : 0;
      if (r < bs) req_pos[r] = base + before;
      // every lane has read its slot's total before the first lanes advance it
      __builtin_amdgcn_wave_barrier();
      if (r < bs && first) running[a] = base + group;
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();

  // 4. Permutation: sorted position -> token.
  for (int64_t t0 = 0; t0 < s; t0 += kPlanThreads) {
    const int t = static_cast<int>(t0) + tid;
    if (t < s) {
      int lo = 0, hi = bs;  // request r with req_ptr[r] <= t < req_ptr[r + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (req_ptr[mid] <= t) lo = mid;
        else hi = mid;
      }
      perm[req_pos[lo] + (t - req_ptr[lo])] = t;
    }
  }

  // 5. Segments and work segments of each slot, padding, tables.
  for (int a = tid; a < L; a += kPlanThreads) {
    const int n = count[a];
    if (n == 0) continue;
    const int segs = (n + chunk - 1) / chunk;
    const int pos0 = first_pos[a];
    int i = first_seg[a];
    for (int q = 0; q < segs; ++q, ++i) {
      const int end = q < segs - 1 ? (q + 1) * chunk : n;
      seg_slots[i] = a;
      seg_indptr[i + 1] = pos0 + end;
    }
    atomicMax(&longest, n < chunk ? n : chunk);
    int w = first_work[a];
    for (int q = 0; q < segs; ++w) {
      int tok = 0;
      int q1 = q;
      while (q1 < segs) {
        const int len = q1 < segs - 1 ? chunk : n - (segs - 1) * chunk;
        if (q1 > q && tok + len > cap) break;
        tok += len;
        ++q1;
      }
      work_slots[w] = a;
      work_indptr[w + 1] = pos0 + (q1 < segs ? q1 * chunk : n);
      atomicMax(&longest_work, tok);
      q = q1;
    }
  }
  for (int64_t i = n_seg + tid; i < p.seg_capacity; i += kPlanThreads) {
    seg_slots[i] = 0;
    seg_indptr[i + 1] = static_cast<int32_t>(s);
  }
  for (int64_t i = n_work + tid; i < p.seg_capacity; i += kPlanThreads) {
    work_slots[i] = 0;
    work_indptr[i + 1] = static_cast<int32_t>(s);
  }
  for (int a = tid; a < L; a += kPlanThreads) {
    ranks_out[a] = p.ranks[a];
    scal_out[a] = __float_as_int(p.scalings[a]);
  }
  if (tid == 0) {
    seg_indptr[0] = 0;
    work_indptr[0] = 0;
  }
  __syncthreads();
  if (tid == 0) {
    p.info[0] = static_cast<int32_t>(n_seg);
    p.info[1] = chunk;
    p.info[2] = longest;
    p.info[3] = static_cast<int32_t>(s);
    p.info[4] = static_cast<int32_t>(n_work);
    p.info[5] = longest_work;
    p.info[6] = SGG_OK;
  }
}

}  // namespace

hipError_t launch_plan_device(const int32_t* seq_lens, const int32_t* req_slots, int32_t bs,
                              const int32_t* ranks, const float* scalings, int32_t L,
                              int32_t is_decode, int32_t max_chunk, int32_t chunk_override,
                              int64_t token_capacity, int32_t seg_capacity, const int64_t* off,
                              int32_t* plan, int32_t* info, hipStream_t stream) {
  DevicePlanParams p{};
  p.seq_lens = seq_lens;
  p.req_slots = req_slots;
  p.ranks = ranks;
  p.scalings = scalings;
  p.plan = plan;
  p.info = info;
  for (int i = 0; i < SGG_PLAN_REGIONS; ++i) p.off[i] = off[i];
  p.token_capacity = token_capacity;
  p.bs = bs;
  p.L = L;
  p.is_decode = is_decode;
  p.max_chunk = max_chunk;
  p.chunk_override = chunk_override;
  p.seg_capacity = seg_capacity;
  hipLaunchKernelGGL(plan_device_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sgg
