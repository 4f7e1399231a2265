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
//
// Optionally (library option "shrink_valu") the kernel takes 16-token tiles
// and computes the tiles of segments' short ends (at most 4 tokens, e.g. the
// one-request segments of a many-adapter decode batch) on the VALU with
// cross-lane reductions instead of MFMA (shrink_tile.h); it reads the same
// bytes.  Measured, it is no faster, so it is off by default.
#include "sgg_device.h"
#include "sgg_internal.h"
#include "sgg_kernels.h"
#include "shrink_tile.h"

namespace sgg {

namespace {

template <int MF, int NF, bool VALU>
__global__ __launch_bounds__(256, 1) void shrink_kernel(ShrinkParams p) {
  __shared__ __attribute__((aligned(16))) char smem[detail::ShrinkShape<MF, NF>::SMEM];
  __shared__ int last_flag;
  int seg, item;
  if (!detail::shrink_item_of(p, blockIdx.x, &seg, &item)) return;
  detail::shrink_tile<MF, NF, VALU>(p, seg, item, smem, &last_flag);
}

template <int MF, int NF, bool VALU = false>
hipError_t launch_mn(const ShrinkParams& p, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL((shrink_kernel<MF, NF, VALU>), dim3(static_cast<unsigned>(grid)), dim3(256),
                     0, stream, p);
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

hipError_t launch_shrink(const ShrinkParams& p, const ShrinkTiling& t, hipStream_t stream) {
  if (t.grid <= 0) return hipSuccess;
  if (t.gemm) return launch_shrink_gemm(p, t.bm, t.bn, t.grid, stream);
  if (t.valu) {
    if (t.mf != 1) return hipErrorInvalidValue;
    switch (t.nf) {
      case 1: return launch_mn<1, 1, true>(p, t.grid, stream);
      case 2: return launch_mn<1, 2, true>(p, t.grid, stream);
      case 3: return launch_mn<1, 3, true>(p, t.grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (t.mf) {
    case 1: return launch_m<1>(p, t.nf, t.grid, stream);
    case 2: return launch_m<2>(p, t.nf, t.grid, stream);
    case 4: return launch_m<4>(p, t.nf, t.grid, stream);
    case 8: return launch_m<8>(p, t.nf, t.grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sgg
