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
//   1. request boundaries (a block-wide scan of the lengths; in decode mode
//      the index itself), validation;
//   2. tokens per slot (LDS histogram), the chunk size, each slot's first
//      sorted position and first segment (scans over the slots: across the
//      lanes of one wave when there are at most 64 slots, of two when there
//      are at most 128);
//   3. each request's first sorted position: the stable counting sort.  For
//      one-token requests every wave places 64 at once (slots matched by one
//      ballot per slot bit, a per-wave count table for the offsets); else one
//      wave walks the requests 64 at a time and, for each slot among them (by
//      ballot), its lanes add the lengths of its earlier lanes to the slot's
//      running position, which the slot's first lane then advances;
//   4. the permutation: one thread per request when every request has one
//      token, else one wave per request writing its tokens' sorted positions;
//   5. segments (full chunks, remainder last) and work segments
//      (consecutive segments of one slot merged greedily within
//      max(chunk, 128) tokens, in closed form), one per thread; capacity
//      padding (slot 0, zero length) and the rank / scaling tables.
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
constexpr int kPlanWaves = kPlanThreads / 64;

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
  // MoE routing (the ROUTE instance, decode mode): request m is top-k copy m
  // and its slot the copy's virtual expert (moe_virtual_slot over these
  // fields); ranks / scalings are the route_L adapters' tables, and the plan's
  // tables those of the L = route_L * route_E + 1 virtual slots (adapter
  // v / route_E for v < route_L * route_E, rank 0 and scaling 0 for the last).
  const int32_t* route_topk;
  const int32_t* route_req_indptr;
  const int32_t* route_req_slots;
  int32_t route_bs, route_top_k, route_E, route_L;
};

__device__ __forceinline__ int chunk_for(int64_t n, int max_chunk) {
  if (max_chunk <= SGG_MIN_CHUNK_SIZE) return SGG_MIN_CHUNK_SIZE;
  const int wanted = n >= 256 ? 128 : (n >= 64 ? 32 : 16);
  return wanted < max_chunk ? wanted : max_chunk;
}

// Exclusive scans of two values over the workgroup: *pa, *pb get the
// prefixes and *ta, *tb the totals.  Every thread must call it.
__device__ void block_exclusive_scan2(int64_t a, int64_t b, int64_t (*wave_sums)[2], int64_t* pa,
                                      int64_t* pb, int64_t* ta, int64_t* tb) {
  constexpr int kWaves = kPlanWaves;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t x = a, y = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(x, d, 64);
    const int64_t v = __shfl_up(y, d, 64);
    if (lane >= d) {
      x += u;
      y += v;
    }
  }
  if (lane == 63) {
    wave_sums[wave][0] = x;
    wave_sums[wave][1] = y;
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan of the wave sums in the first wave
    int64_t sx = lane < kWaves ? wave_sums[lane][0] : 0;
    int64_t sy = lane < kWaves ? wave_sums[lane][1] : 0;
    const int64_t ox = sx, oy = sy;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const int64_t u = __shfl_up(sx, d, 64);
      const int64_t v = __shfl_up(sy, d, 64);
      if (lane >= d) {
        sx += u;
        sy += v;
      }
    }
    if (lane < kWaves) {
      wave_sums[lane][0] = sx - ox;
      wave_sums[lane][1] = sy - oy;
    }
    if (lane == kWaves - 1) {
      wave_sums[kWaves][0] = sx;
      wave_sums[kWaves][1] = sy;
    }
  }
  __syncthreads();
  *pa = wave_sums[wave][0] + x - a;
  *pb = wave_sums[wave][1] + y - b;
  *ta = wave_sums[kWaves][0];
  *tb = wave_sums[kWaves][1];
  __syncthreads();  // the sums are read before a later call overwrites them
}

// Inclusive scans of three values over one wave (32-bit, wrapping).
__device__ __forceinline__ void wave_inclusive_scan3(uint32_t& x, uint32_t& y, uint32_t& z) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = __shfl_up(x, d, 64);
    const uint32_t v = __shfl_up(y, d, 64);
    const uint32_t w = __shfl_up(z, d, 64);
    if (lane >= d) {
      x += u;
      y += v;
      z += w;
    }
  }
}

// The work segments of one slot of n tokens: its segments are full chunks
// and a remainder r = n % chunk (if any); merging consecutive segments
// greedily within `cap` tokens gives groups of m = cap / chunk full chunks,
// and the remainder joins the last group when it still fits.
struct SlotWork {
  int nf, r, m, full_groups, merged, groups, longest;
};

__device__ __forceinline__ SlotWork slot_work(int n, int chunk, int cap) {
  SlotWork w;
  w.nf = n / chunk;
  w.r = n - w.nf * chunk;
  w.m = cap / chunk > 0 ? cap / chunk : 1;
  w.full_groups = (w.nf + w.m - 1) / w.m;
  const int last_full = w.nf == 0 ? 0 : (w.nf % w.m == 0 ? w.m : w.nf % w.m);
  w.merged = w.r > 0 && w.nf > 0 && last_full * chunk + w.r <= cap;
  w.groups = w.full_groups + (w.r > 0 && !w.merged ? 1 : 0);
  int lw = (w.nf >= w.m ? w.m : w.nf) * chunk;  // a full group
  const int tail = last_full * chunk + (w.merged ? w.r : 0);
  if (tail > lw) lw = tail;
  if (w.r > 0 && !w.merged && w.r > lw) lw = w.r;
  w.longest = n == 0 ? 0 : lw;
  return w;
}

// Token offset (within its slot) where work segment g of the slot ends.
__device__ __forceinline__ int slot_work_end(const SlotWork& w, int g, int n, int chunk) {
  if (g < w.full_groups - 1) return (g + 1) * w.m * chunk;
  if (g == w.full_groups - 1) return w.merged ? n : w.nf * chunk;
  return n;  // the remainder on its own
}

// Largest index a < n with v[a] <= x (v non-decreasing, v[0] <= x).
__device__ __forceinline__ int last_at_most(const int32_t* v, int n, int x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (v[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <bool ROUTE>
__global__ __launch_bounds__(kPlanThreads) void plan_device_kernel(DevicePlanParams p) {
  __shared__ int32_t count[kDevicePlanMaxLoras];      // tokens per slot
  __shared__ int32_t first_pos[kDevicePlanMaxLoras];  // first sorted position per slot
  __shared__ int32_t running[kDevicePlanMaxLoras];    // next sorted position per slot
  __shared__ int32_t first_seg[kDevicePlanMaxLoras];  // first segment per slot
  __shared__ int32_t first_work[kDevicePlanMaxLoras]; // first work segment per slot
  __shared__ int32_t req_ptr[kDevicePlanMaxReqs + 1]; // request token boundaries
  __shared__ int32_t req_pos[kDevicePlanMaxReqs];     // first sorted position per request
  __shared__ uint16_t wave_count[kPlanWaves * kDevicePlanMaxLoras];  // step 3, one-token requests
  __shared__ int64_t wave_sums[kPlanThreads / 64 + 1][2];
  __shared__ int32_t status, longest, longest_work, all_unit;
  __shared__ uint32_t slot_totals[2];
  __shared__ uint32_t wave0_totals[3];  // step 2, 65-128 slots

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
    all_unit = 1;
  }
  if (tid < L) count[tid] = 0;
  // the rank and scaling tables, requested now so that their round trip
  // overlaps the planning (written out in step 5; L <= kPlanThreads)
  int32_t rank_of_tid = 0, scal_of_tid = 0;
  if constexpr (ROUTE) {
    if (tid < L - 1) {
      rank_of_tid = p.ranks[tid / p.route_E];
      scal_of_tid = __float_as_int(p.scalings[tid / p.route_E]);
    }
  } else if (tid < L) {
    rank_of_tid = p.ranks[tid];
    scal_of_tid = __float_as_int(p.scalings[tid]);
  }
  __syncthreads();

  // 1. Request boundaries and validation; tokens per slot.
  int64_t carry = 0;
  for (int r0 = 0; r0 < bs; r0 += kPlanThreads) {
    const int r = r0 + tid;
    int len = 0;
    if (r < bs) {
      len = p.seq_lens ? p.seq_lens[r] : 1;
      const int a = ROUTE ? moe_virtual_slot(p.route_req_indptr, p.route_req_slots, p.route_bs,
                                             p.route_topk, p.route_top_k, p.route_E,
                                             p.route_L, r)
                          : p.req_slots[r];
      if (len < 0 || (p.is_decode && len != 1)) atomicOr(&status, 1);
      if (a < 0 || a >= L) atomicOr(&status, 2);
      else if (len > 0) atomicAdd(&count[a], len);
      if (len != 1) all_unit = 0;
      req_slots_out[r] = a;
      req_pos[r] = a;  // the slot, until step 3 replaces it with the position
    }
    int64_t pre, unused, chunk_total, unused_total;
    if (p.seq_lens == nullptr) {  // one token per request: the prefix is the index
      pre = r - r0;
      chunk_total = bs - r0 < kPlanThreads ? bs - r0 : kPlanThreads;
    } else {
      block_exclusive_scan2(len > 0 ? len : 0, 0, wave_sums, &pre, &unused, &chunk_total,
                            &unused_total);
    }
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
  const SlotWork sw = slot_work(n_slot > 0 ? n_slot : 0, chunk, cap);
  const int works = n_slot > 0 ? sw.groups : 0;
  if (n_slot > 0) {
    atomicMax(&longest, n_slot < chunk ? n_slot : chunk);
    atomicMax(&longest_work, sw.longest);
  }
  int64_t n_seg, n_work;
  if (L <= 64) {
    // The slots fit the first wave: 32-bit scans across its lanes, no
    // block-level pass.  (The sums can wrap only for a batch of more than
    // 2^31 tokens, which the status already rejects.)
    if (wave == 0) {
      uint32_t x = static_cast<uint32_t>(n_slot), y = static_cast<uint32_t>(segs);
      uint32_t z = static_cast<uint32_t>(works);
      wave_inclusive_scan3(x, y, z);
      if (tid < L) {
        first_pos[tid] = static_cast<int32_t>(x - static_cast<uint32_t>(n_slot));
        first_seg[tid] = static_cast<int32_t>(y - static_cast<uint32_t>(segs));
        first_work[tid] = static_cast<int32_t>(z - static_cast<uint32_t>(works));
      }
      const uint32_t ty = __shfl(y, 63, 64), tz = __shfl(z, 63, 64);
      if (lane == 0) {
        slot_totals[0] = ty;
        slot_totals[1] = tz;
        if (static_cast<int64_t>(ty) > p.seg_capacity) atomicOr(&status, 8);
      }
    }
    __syncthreads();
    n_seg = slot_totals[0];
    n_work = slot_totals[1];
  } else if (L <= 128) {
    // The slots fit the first two waves: each scans its 64 slots, then wave
    // 1 adds wave 0's totals (one barrier; no block-level pass).
    uint32_t x = static_cast<uint32_t>(n_slot), y = static_cast<uint32_t>(segs);
    uint32_t z = static_cast<uint32_t>(works);
    if (wave < 2) {
      wave_inclusive_scan3(x, y, z);
      if (wave == 0 && lane == 63) {
        wave0_totals[0] = x;
        wave0_totals[1] = y;
        wave0_totals[2] = z;
      }
    }
    __syncthreads();
    if (wave == 1) {
      x += wave0_totals[0];
      y += wave0_totals[1];
      z += wave0_totals[2];
    }
    if (wave < 2) {
      if (tid < L) {
        first_pos[tid] = static_cast<int32_t>(x - static_cast<uint32_t>(n_slot));
        first_seg[tid] = static_cast<int32_t>(y - static_cast<uint32_t>(segs));
        first_work[tid] = static_cast<int32_t>(z - static_cast<uint32_t>(works));
      }
      if (wave == 1 && lane == 63) {
        slot_totals[0] = y;
        slot_totals[1] = z;
        if (static_cast<int64_t>(y) > p.seg_capacity) atomicOr(&status, 8);
      }
    }
    __syncthreads();
    n_seg = slot_totals[0];
    n_work = slot_totals[1];
  } else {
    // one scan of the token counts, one of the segment and work-segment
    // counts packed in one word (each total stays below 2^31)
    int64_t pos, packed, tot_tok, tot_packed;
    block_exclusive_scan2(n_slot, (static_cast<int64_t>(segs) << 32) | works, wave_sums, &pos,
                          &packed, &tot_tok, &tot_packed);
    const int64_t sg = packed >> 32, wk = packed & 0xffffffffll;
    n_seg = tot_packed >> 32;
    n_work = tot_packed & 0xffffffffll;
    if (tid < L) {
      first_pos[tid] = static_cast<int32_t>(pos);
      first_seg[tid] = static_cast<int32_t>(sg);
      first_work[tid] = static_cast<int32_t>(wk);
    }
    if (tid == 0 && n_seg > p.seg_capacity) atomicOr(&status, 8);
    __syncthreads();
  }
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
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int slot_bits = L > 1 ? 32 - __builtin_clz(static_cast<unsigned>(L - 1)) : 0;
  if (all_unit) {
    // One-token requests (decode batches, MoE copies), kPlanThreads at a
    // time, every wave at once.  A wave finds the lanes of each lane's slot
    // by matching the slot's bits, one ballot per bit (whatever the number
    // of slots among its 64); the slot's first lane records the wave's count
    // in a per-wave table, and a lane's position is the slot's running
    // position plus the counts of the earlier waves plus its rank in its
    // wave.  Then one thread per slot advances the running position.
    for (int r0 = 0; r0 < bs; r0 += kPlanThreads) {
      for (int i = tid; i < kPlanWaves * L; i += kPlanThreads) wave_count[i] = 0;
      __syncthreads();
      const int r = r0 + tid;
      const bool valid = r < bs;
      const int a = valid ? req_pos[r] : -1;
      uint64_t same = __ballot(valid);
      for (int b = 0; b < slot_bits; ++b) {
        const bool bit = (a >> b) & 1;
        const uint64_t ones = __ballot(valid && bit);
        same &= bit ? ones : ~ones;
      }
      const int rank = __popcll(same & below);
      if (valid && rank == 0) wave_count[wave * L + a] = static_cast<uint16_t>(__popcll(same));
      __syncthreads();
      if (valid) {
        int pos = running[a] + rank;
        for (int w = 0; w < wave; ++w) pos += wave_count[w * L + a];
        req_pos[r] = pos;
      }
      __syncthreads();
      for (int a2 = tid; a2 < L; a2 += kPlanThreads) {
        int t = 0;
        for (int w = 0; w < kPlanWaves; ++w) t += wave_count[w * L + a2];
        running[a2] += t;
      }
      __syncthreads();
    }
  } else if (tid < 64) {
    // One wave, 64 requests at a time.  For each slot present among them
    // (in order of first appearance): its lanes' positions are the slot's
    // running position plus the lengths of its earlier lanes.
    for (int r0 = 0; r0 < bs; r0 += 64) {
      const int r = r0 + lane;
      const bool valid = r < bs;
      const int a = valid ? req_pos[r] : -1;
      const int len = valid ? req_ptr[r + 1] - req_ptr[r] : 0;
      uint64_t todo = __ballot(valid);
      while (todo != 0) {
        const int leader = __builtin_ctzll(todo);
        const int slot = __builtin_amdgcn_readlane(a, leader);
        const uint64_t m = __ballot(a == slot);
        // exclusive scan of the members' lengths
        int v = (a == slot) ? len : 0;
        const int own = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int u = __shfl_up(v, d, 64);
          if (lane >= d) v += u;
        }
        const int before = v - own;
        const int total = __shfl(v, 63, 64);
        const int base = running[slot];
        if (a == slot) req_pos[r] = base + before;
        __builtin_amdgcn_wave_barrier();
        if (lane == leader) running[slot] = base + total;
        __builtin_amdgcn_wave_barrier();
        todo &= ~m;
      }
    }
  }
  __syncthreads();

  // 4. Permutation: sorted position -> token; one thread per request when
  // every request has one token (decode), else one wave per request, its
  // lanes writing consecutive positions.
  if (all_unit) {
    for (int r = tid; r < bs; r += kPlanThreads) perm[req_pos[r]] = req_ptr[r];
  } else {
    for (int r = wave; r < bs; r += kPlanWaves) {
      const int start = req_ptr[r];
      const int len = req_ptr[r + 1] - start;
      const int pos = req_pos[r];
      for (int k = lane; k < len; k += 64) perm[pos + k] = start + k;
    }
  }

  // 5. Segments and work segments (one per thread, each finding its slot by
  // binary search over the slots' first indices), padding, tables.
  for (int i = tid; i < n_seg; i += kPlanThreads) {
    const int a = last_at_most(first_seg, L, i);
    const int q = i - first_seg[a];
    const int n = count[a];
    const int end = (q + 1) * chunk < n ? (q + 1) * chunk : n;
    seg_slots[i] = a;
    seg_indptr[i + 1] = first_pos[a] + end;
  }
  for (int w = tid; w < n_work; w += kPlanThreads) {
    const int a = last_at_most(first_work, L, w);
    const int n = count[a];
    const SlotWork sa = slot_work(n, chunk, cap);
    work_slots[w] = a;
    work_indptr[w + 1] = first_pos[a] + slot_work_end(sa, w - first_work[a], n, chunk);
  }
  for (int64_t i = n_seg + tid; i < p.seg_capacity; i += kPlanThreads) {
    seg_slots[i] = 0;
    seg_indptr[i + 1] = static_cast<int32_t>(s);
  }
  for (int64_t i = n_work + tid; i < p.seg_capacity; i += kPlanThreads) {
    work_slots[i] = 0;
    work_indptr[i + 1] = static_cast<int32_t>(s);
  }
  if (tid < L) {
    ranks_out[tid] = rank_of_tid;
    scal_out[tid] = scal_of_tid;
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
  hipLaunchKernelGGL(plan_device_kernel<false>, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_moe_plan(const MoeRouteParams& r, int32_t max_chunk, int32_t seg_capacity,
                           const int64_t* off, int32_t* plan, int32_t* info, hipStream_t stream) {
  DevicePlanParams p{};
  p.seq_lens = nullptr;
  p.req_slots = nullptr;
  p.ranks = r.ranks;
  p.scalings = r.scalings;
  p.plan = plan;
  p.info = info;
  for (int i = 0; i < SGG_PLAN_REGIONS; ++i) p.off[i] = off[i];
  p.token_capacity = r.copies;
  p.bs = static_cast<int32_t>(r.copies);
  p.L = r.L * r.E + 1;
  p.is_decode = 1;
  p.max_chunk = max_chunk;
  p.chunk_override = 0;
  p.seg_capacity = seg_capacity;
  p.route_topk = r.topk_ids;
  p.route_req_indptr = r.req_seg_indptr;
  p.route_req_slots = r.req_weight_indices;
  p.route_bs = r.bs;
  p.route_top_k = r.top_k;
  p.route_E = r.E;
  p.route_L = r.L;
  hipLaunchKernelGGL(plan_device_kernel<true>, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sgg
