"""MoE LoRA oracle: per-request routing to virtual experts and the LoRA add
on a fused-MoE intermediate, in float64.

Test infrastructure only (see the package docstring).

Source: the PR #24007 report page ("implementation breakdown", items 2-4).
The chunked backend's segments are cut per adapter across requests, so a
MoE layer cannot recover a token's adapter from them; the batch therefore
also carries per-request routing: ``req_seg_indptr`` (bs + 1 token
boundaries of the requests, in the batch's token order) and
``req_weight_indices`` (bs adapter slots), which ``_get_lora_info`` prefers
over the segment arrays.  The MoE LoRA kernel that consumes them
(``merged_experts_fused_moe_lora_add``) is named there but its body is not
given.  Reading used here, the plainest one the report supports:

* token t lies in request r(t): req_seg_indptr[r] <= t < req_seg_indptr[r+1];
  its adapter is a(t) = req_weight_indices[r(t)];
* the router picked experts topk_ids[t][0..k-1] for it; copy j of token t
  goes to the virtual expert v = a(t) * E + topk_ids[t][j] (E experts);
* the LoRA weights of adapter a on expert e are A[a][e] (R x K) and
  B[a][e] (N x R), rank rho = lora_ranks[a], scaling sigma = scalings[a];
* the add targets the fused-MoE intermediate, one row per copy, row
  m = t * k + j:
      out[m] += sigma * sum_{i < rho} B[a][e][:, i] * (sum_q A[a][e][i][q] x[t][q])
  A slot of rank 0 (the base model) leaves its rows unchanged.

All arithmetic is float64 on inputs the caller has upcast exactly.
"""

import numpy as np


def token_requests(req_seg_indptr, num_tokens):
    """r(t) for every token t: the request whose [start, end) holds it."""
    out = np.full(num_tokens, -1, dtype=np.int64)
    for r in range(len(req_seg_indptr) - 1):
        for t in range(int(req_seg_indptr[r]), int(req_seg_indptr[r + 1])):
            out[t] = r
    return out


def virtual_experts(req_seg_indptr, req_weight_indices, topk_ids, num_experts):
    """v[t * k + j] = a(t) * E + topk_ids[t][j], a(t) from the per-request
    routing fields (PR #24007 report: _get_lora_info reads them)."""
    topk_ids = np.asarray(topk_ids, dtype=np.int64)
    s, k = topk_ids.shape
    req = token_requests(req_seg_indptr, s)
    v = np.empty(s * k, dtype=np.int64)
    for t in range(s):
        a = int(req_weight_indices[req[t]])
        for j in range(k):
            v[t * k + j] = a * num_experts + int(topk_ids[t, j])
    return v


def moe_lora_add(x, A, B, out, req_seg_indptr, req_weight_indices, topk_ids, lora_ranks,
                 scalings):
    """out (s*k, N) after the MoE LoRA add; x (s, K), A (L, E, R, K),
    B (L, E, N, R).  Returns a new array; `out` is not modified."""
    x = np.asarray(x, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    y = np.array(out, dtype=np.float64, copy=True)
    topk_ids = np.asarray(topk_ids, dtype=np.int64)
    s, k = topk_ids.shape
    req = token_requests(req_seg_indptr, s)
    for t in range(s):
        a = int(req_weight_indices[req[t]])
        rho = int(lora_ranks[a])
        if rho == 0:
            continue
        sigma = float(scalings[a])
        for j in range(k):
            e = int(topk_ids[t, j])
            h = A[a, e, :rho, :] @ x[t]              # rank-rho LoRA-A of expert e
            y[t * k + j] += sigma * (B[a, e, :, :rho] @ h)
    return y
