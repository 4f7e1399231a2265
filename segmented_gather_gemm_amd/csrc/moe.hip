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
// One thread per copy: the token's request -- request t itself when it holds
// token t (one-token requests: one round trip), else by binary search over
// the request boundaries -- then the virtual expert; copies whose request, adapter
// or expert is out of range go to the extra virtual slot L*E, whose rank is 0
// (the kernels leave such rows unchanged).  The first L*E + 1 threads also
// write the virtual rank and scaling tables (adapter a's values for every
// expert).
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
  const int64_t t = m / p.top_k;
  const int e = p.topk_ids[m];
  // the request holding token t: the last r with req_seg_indptr[r] <= t,
  // valid if t also lies before its end.  Request t itself when it holds the
  // token (then it is that last r); else a binary search.
  int r = -1;
  if (t < p.bs && p.req_seg_indptr[t] <= t && t < p.req_seg_indptr[t + 1]) {
    r = static_cast<int>(t);
  } else {
    int lo = 0, hi = p.bs;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.req_seg_indptr[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    if (lo < p.bs && p.req_seg_indptr[lo] <= t && t < p.req_seg_indptr[lo + 1]) r = lo;
  }
  int v = static_cast<int>(nv);
  if (r >= 0) {
    const int a = p.req_weight_indices[r];
    if (a >= 0 && a < p.L && e >= 0 && e < p.E) v = a * p.E + e;
  }
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
