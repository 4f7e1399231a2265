// The stacked LoRA call -- shrink, then expand with the same plan
// (chunked_backend.py page: run_qkv_lora / run_gate_up_lora) -- in one
// launch, for the batches the split-K shrink serves (decode-sized batches).
//
// The pages launch the shrink and then the expand.  For a decode batch each
// of the two moves a few megabytes, about what one launch costs to ramp up
// and drain, so here one grid holds both.  Producer blocks [0, Gs) are the
// split-K shrink tiles (16 tokens x 16 rank rows over one K range), which
// leave f32 partials in the workspace exactly as in the two-launch call.
// Consumer blocks [Gs, Gs + Ge) are the expand tiles: each requests its B
// fragments, waits until every producer block of its segment has published,
// then sums the partials in split order while staging h.  That is the
// arithmetic of the two-launch call, so both give the same bits.
//
// Progress.  Producers never wait and come first in the grid, and each XCD
// dispatches its blocks in order, so every producer is placed before any
// consumer that could wait for it; the host also takes this launch only
// when the whole grid fits on the device at once.  The wait is bounded all
// the same: after `spin_limit` polls a consumer gives up, computes its
// segment's producer tiles itself (the same partials, written again) and
// sets bit 0 of the status word, so every block always exits.
//
// Hand-off word, one per segment: bits 0-15 count producers that have
// published, bits 16-30 count blocks (producers and consumers) that are done
// with the word.  The partials go out as device-coherent stores; a producer
// adds to both fields at once after every one of its waves has waited for its
// own stores and the workgroup barrier (wave_stores_done).  A consumer polls
// bits 0-15 and then reads the partials with device-coherent loads; when it
// is done it adds to bits 16-30.  The block that completes the count resets
// the word to zero for the next call.  All arrivals are RMWs on the one word,
// so the reset comes after every other block's use of it.
#include <mutex>

#include "sgg_device.h"
#include "sgg_internal.h"
#include "sgg_kernels.h"
#include "expand_tile.h"
#include "shrink_tile.h"

namespace sgg {

namespace {

constexpr int kDoneUnit = 1 << 16;

// One block of segment `seg` is done with its hand-off word (thread 0 only);
// the last of all the segment's blocks resets it.  `add` also carries a
// producer's ready count.
__device__ __forceinline__ void arrive(const FusedSync& fs, int seg, int add) {
  int32_t* word = fs.ready + seg;
  const int total = fs.producers_per_seg + fs.consumers_per_seg;
  const int old = __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((old >> 16) == total - 1)
    __hip_atomic_store(word, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MF, int NF, int KS>
struct FusedShape {
  static constexpr int A = detail::ShrinkShape<MF, NF>::SMEM;
  static constexpr int B = detail::ExpandShape<1, KS>::SMEM;
  static constexpr int SMEM = A > B ? A : B;
};

// Producer tiles of 16*MF tokens x 16*NF rank rows; consumer tiles of 128
// columns with rank steps KS.
// Block timeline record (FusedSync::trace): lanes 0-3 of wave 0 each store
// one word, with vector stores.
__device__ __forceinline__ void trace_block(const FusedSync& fs, uint64_t t0, uint64_t t1,
                                            int role) {
  const int b = blockIdx.x;
  if (fs.trace == nullptr || b >= fs.trace_blocks || threadIdx.x >= 4) return;
  const uint64_t t2 = __builtin_amdgcn_s_memrealtime();
  const int i = threadIdx.x;
  const uint64_t v = i == 0 ? t0 : i == 1 ? t1 : i == 2 ? t2 : static_cast<uint64_t>(role);
  fs.trace[4 * static_cast<int64_t>(b) + i] = v;
}

template <int MF, int NF, int KS>
__global__ __launch_bounds__(256) void fused_kernel(ShrinkParams ps, ExpandParams pe,
                                                    FusedSync fs) {
  __shared__ __attribute__((aligned(16))) char smem[FusedShape<MF, NF, KS>::SMEM];
  __shared__ int unused_flag;
  __shared__ int published;
  const uint64_t t_start = fs.trace ? __builtin_amdgcn_s_memrealtime() : 0;
  const int b = blockIdx.x;
  if (b < fs.producer_blocks) {
    int seg, item;
    if (!detail::shrink_item_of(ps, b, &seg, &item)) return;
    detail::shrink_tile<MF, NF>(ps, seg, item, smem, &unused_flag);
    wave_stores_done();
    __syncthreads();
    const uint64_t t_work = fs.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    if (threadIdx.x == 0) arrive(fs, seg, 1 + kDoneUnit);
    trace_block(fs, t_start, t_work, 0);
    return;
  }
  int seg, tile;
  if (!detail::expand_item_of(pe, b - fs.producer_blocks, &seg, &tile)) return;
  uint64_t t_wait = 0;
  int role = 1;
  const auto wait = [&]() {
    if (threadIdx.x == 0) {
      int ok = 0;
      for (int64_t n = 0;; ++n) {
        const int v = __hip_atomic_load(fs.ready + seg, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
        if ((v & (kDoneUnit - 1)) >= fs.producers_per_seg) {
          ok = 1;
          break;
        }
        if (n >= fs.spin_limit) break;
        __builtin_amdgcn_s_sleep(2);
      }
      published = ok;
    }
    __syncthreads();
    if (fs.trace) t_wait = __builtin_amdgcn_s_memrealtime();
    if (published) return false;
    role = 2;
    // Gave up: make this segment's partials here (the same values the
    // producers write), then read them as usual.
    if (threadIdx.x == 0)
      __hip_atomic_fetch_or(fs.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0; it < fs.producers_per_seg; ++it) {
      detail::shrink_tile<MF, NF>(ps, seg, it, smem, &unused_flag);
      __syncthreads();
    }
    wave_stores_done();
    __syncthreads();
    return true;
  };
  detail::expand_tile<1, KS, true, true>(pe, seg, tile, smem, wait);
  __syncthreads();
  if (threadIdx.x == 0) arrive(fs, seg, kDoneUnit);
  trace_block(fs, t_start, t_wait, role);
}

#define SGG_FUSED_INSTANCES(X)                                                    \
  X(1, 1, 1) X(1, 2, 1) X(1, 3, 1) X(2, 1, 1) X(2, 2, 1) X(2, 3, 1)               \
  X(4, 1, 1) X(4, 2, 1) X(4, 3, 1)                                                \
  X(1, 1, 2) X(1, 2, 2) X(1, 3, 2) X(2, 1, 2) X(2, 2, 2) X(2, 3, 2)               \
  X(4, 1, 2) X(4, 2, 2) X(4, 3, 2)

constexpr int fused_key(int mf, int nf, int ks) { return (mf * 4 + nf) * 4 + ks; }

const void* fused_for(int mf, int nf, int ks) {
  switch (fused_key(mf, nf, ks)) {
#define SGG_FN(M, N, K) \
    case fused_key(M, N, K): return reinterpret_cast<const void*>(&fused_kernel<M, N, K>);
    SGG_FUSED_INSTANCES(SGG_FN)
#undef SGG_FN
    default: return nullptr;
  }
}

constexpr int kMaxDevices = 64;
std::mutex g_resident_mutex;
int64_t g_resident[kMaxDevices][64] = {};   // (device, fused_key) -> blocks; 0 unknown

}  // namespace

int64_t fused_resident_blocks(int mf, int nf, int ks) {
  const void* fn = fused_for(mf, nf, ks);
  int dev = -1;
  if (fn == nullptr || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  const int key = fused_key(mf, nf, ks);
  std::lock_guard<std::mutex> lock(g_resident_mutex);
  if (g_resident[dev][key] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    g_resident[dev][key] = static_cast<int64_t>(per_cu) * cus;
  }
  return g_resident[dev][key];
}

hipError_t launch_fused(const ShrinkParams& ps, const ShrinkTiling& ts, const ExpandParams& pe,
                        const ExpandTiling& te, const FusedSync& fs, hipStream_t stream) {
  if (ts.gemm || ts.ksplit < 1 || te.pairs != 1) return hipErrorInvalidValue;
  const int64_t grid = ts.grid + te.grid;
  if (grid <= 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(grid)), b(256);
  switch (fused_key(ts.mf, ts.nf, te.ks)) {
#define SGG_LAUNCH(M, N, K)                                                              \
    case fused_key(M, N, K):                                                             \
      hipLaunchKernelGGL((fused_kernel<M, N, K>), g, b, 0, stream, ps, pe, fs); break;
    SGG_FUSED_INSTANCES(SGG_LAUNCH)
#undef SGG_LAUNCH
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sgg
