// Per-request routing for the MoE LoRA add (PR #24007 report page,
// implementation breakdown items 2-4): the chunked plan cuts its segments per
// adapter across requests, so a MoE layer finds each token's adapter through
// the per-request fields instead -- req_seg_indptr (the requests' token
// boundaries) and req_weight_indices (their adapter slots).  Here every top-k
// copy (token t, choice j) becomes a one-token request of the "virtual
// expert" v = a(t) * E + topk_ids[t][j]; the chunked planner then sorts and
// segments the copies by virtual expert like any decode batch, and the
// stacked shrink + expand adds each copy's LoRA delta into its row t*k + j of
// the fused-MoE intermediate.
//
// One thread per copy writes its virtual expert (moe_virtual_slot); copies
// whose request, adapter or expert is out of range go to the extra virtual
// slot L*E, whose rank is 0 (the kernels leave such rows unchanged).  The
// first L*E + 1 threads also write the virtual rank and scaling tables
// (adapter a's values for every expert).  lora_moe_plan does the same inside
// the device planner's launch.
#include "sgg_device.h"
#include "sgg_kernels.h"

namespace sgg {

namespace {

__global__ __launch_bounds__(256) void moe_route_kernel(MoeRouteParams p) {
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nv = static_cast<int64_t>(p.L) * p.E;
  if (m <= nv) {
    const int a = static_cast<int>(m / p.E);
    p.vranks[m] = m < nv ? p.ranks[a] : 0;
    p.vscalings[m] = m < nv ? p.scalings[a] : 0.f;
  }
  if (m >= p.copies) return;
  const int v = moe_virtual_slot(p.req_seg_indptr, p.req_weight_indices, p.bs, p.topk_ids,
                                 p.top_k, p.E, p.L, m);
  p.slots[m] = v;
}

}  // namespace

hipError_t launch_moe_route(const MoeRouteParams& p, hipStream_t stream) {
  const int64_t nv = static_cast<int64_t>(p.L) * p.E + 1;
  const int64_t n = p.copies > nv ? p.copies : nv;
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(moe_route_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sgg
