"""Math oracle: per-token LoRA shrink / expand / embedding gather in float64.

Test infrastructure only (see the package docstring).

What is computed, per token t of request r(t) with adapter slot a = slot[r(t)],
rank rho = ranks[a] and scaling sigma = scalings[a]:

* shrink (``run_lora_a_sgemm`` / ``chunked_sgmv_lora_shrink_forward`` on the
  ``chunked_backend.py`` page; shapes from the ``base_backend.py`` page,
  ``run_lora_a_sgemm``: x is (s, in), A is (L, c*r, in), h is (s, c*r)):
      h[t, k*R + j] = sum_q A[a, k*R + j, q] * x[t, q]      for k < c, j < rho
      h[t, k*R + j] = 0                                      for rho <= j < R
* expand (``run_lora_b_sgemm`` / ``run_qkv_lora`` / ``run_gate_up_lora``;
  ``base_backend.py`` page: B is (L, out, r) or stacked (L, sum of widths, r)):
      y[t, o_k + n] = base[t, o_k + n]
                      + sigma * sum_{j < rho} B[a, o_k + n, j] * h[t, k*R + j]
  for every slice k and column n < o_{k+1} - o_k; columns at or beyond o_c
  keep base; a missing base counts as zero.
* embedding (``run_lora_a_embedding``; A_emb is (L, rank, vocab), out (s, rank)):
      e[t, j] = A_emb[a, j, ids[t]]   for j < rho and 0 <= ids[t] < vocab, else 0.

Tokens are request-major (the ``repeat_interleave`` in ``_get_permutation``).
A slot of rank 0 is the base model (``lora_manager.py`` page,
``prepare_lora_batch``: rank 0 and scaling 0 for requests without an adapter),
so its rows of h and e are zero and its output rows equal base exactly.

Readings: only the first rho rows per slice of A and the first rho columns of
B take part (padding beyond rho is never read); h column block k feeds slice k.

All arithmetic is float64 on inputs the caller has upcast exactly (bf16 ->
float64).  No plan, permutation or segment array is read here.
"""

import numpy as np


def request_of_token(seq_lens):
    """Request index of every token, tokens laid out request after request."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    return np.repeat(np.arange(len(seq_lens), dtype=np.int64), seq_lens)


def _rows_by_request(seq_lens, rows):
    """Group the wanted token indices by the request they belong to.

    Yields (request, positions in ``rows``, token indices); positions let the
    caller scatter the per-request results back into ``rows`` order.
    """
    req = request_of_token(seq_lens)
    rows = np.asarray(rows, dtype=np.int64)
    owner = req[rows]
    for r in np.unique(owner):
        pos = np.nonzero(owner == r)[0]
        yield int(r), pos, rows[pos]


def _all_rows(seq_lens, rows):
    if rows is None:
        return np.arange(int(np.sum(seq_lens)), dtype=np.int64)
    return np.asarray(rows, dtype=np.int64)


def shrink(x, A, seq_lens, req_slots, lora_ranks, num_slices, rows=None):
    """LoRA-A for the tokens in ``rows`` (all tokens if None).

    x: (s, K) float64; A: (L, c*R, K) float64.  Returns (len(rows), c*R).
    """
    rows = _all_rows(seq_lens, rows)
    c = num_slices
    R = A.shape[1] // c
    if A.shape[1] != c * R:
        raise ValueError("A rows must be num_slices * R")
    h = np.zeros((len(rows), c * R), dtype=np.float64)
    for r, pos, toks in _rows_by_request(seq_lens, rows):
        a = int(req_slots[r])
        rho = min(int(lora_ranks[a]), R)
        if rho <= 0:
            continue
        xt = x[toks]                                  # (n, K)
        for k in range(c):
            Ak = A[a, k * R:k * R + rho, :]           # (rho, K)
            h[pos, k * R:k * R + rho] = xt @ Ak.T
    return h


def expand(h, B, base, seq_lens, req_slots, lora_ranks, scalings,
           slice_offsets, rows=None):
    """LoRA-B with scaling, added to base, for the tokens in ``rows``.

    h: (len(rows), c*R) rows aligned with ``rows``; B: (L, N, R);
    base: (len(rows), W) with W >= slice_offsets[-1], or None for zeros.
    Returns the new output rows (len(rows), W).
    """
    rows = _all_rows(seq_lens, rows)
    offs = [int(o) for o in slice_offsets]
    c = len(offs) - 1
    R = B.shape[2]
    if h.shape[1] != c * R:
        raise ValueError("h width must be num_slices * R")
    width = offs[-1] if base is None else base.shape[1]
    y = np.zeros((len(rows), width)) if base is None else np.array(base, dtype=np.float64)
    # request grouping over positions 0..len(rows)-1 of the caller's arrays
    for r, pos, _ in _rows_by_request(seq_lens, rows):
        a = int(req_slots[r])
        rho = min(int(lora_ranks[a]), R)
        if rho <= 0:
            continue
        sigma = float(scalings[a])
        for k in range(c):
            Bk = B[a, offs[k]:offs[k + 1], :rho]      # (w_k, rho)
            hk = h[pos, k * R:k * R + rho]            # (n, rho)
            y[pos, offs[k]:offs[k + 1]] += sigma * (hk @ Bk.T)
    return y


def lora_forward(x, A, B, base, seq_lens, req_slots, lora_ranks, scalings,
                 slice_offsets, rows=None):
    """Shrink then expand with the same routing (``run_qkv_lora`` /
    ``run_gate_up_lora``; plain B is one slice with offsets [0, out])."""
    rows = _all_rows(seq_lens, rows)
    c = len(slice_offsets) - 1
    h = shrink(x, A, seq_lens, req_slots, lora_ranks, c, rows)
    return expand(h, B, base, seq_lens, req_slots, lora_ranks, scalings,
                  slice_offsets, rows)


def merged_dense_weight(A, B, a, rho, sigma, slice_offsets):
    """Closed form of one adapter's update as a single dense matrix.

    W[o_k + n, :] = sigma * B[a, o_k + n, :rho] @ A[a, k*R : k*R + rho, :],
    so y = base + W x for every token of that adapter.  Used to pin the
    two-step oracle (association order differs).
    """
    offs = [int(o) for o in slice_offsets]
    c = len(offs) - 1
    R = B.shape[2]
    K = A.shape[2]
    W = np.zeros((offs[-1], K))
    if rho <= 0:
        return W
    for k in range(c):
        W[offs[k]:offs[k + 1]] = sigma * (B[a, offs[k]:offs[k + 1], :rho]
                                          @ A[a, k * R:k * R + rho, :])
    return W


def embedding_a(input_ids, A_emb, seq_lens, req_slots, lora_ranks, vocab_size,
                rows=None):
    """LoRA-A embedding lookup: column ``ids[t]`` of the token's adapter.

    A_emb: (L, R_e, V).  Ids outside [0, vocab_size) give zeros (the chunked
    backend supports no added-vocabulary embeddings).  Returns (len(rows), R_e).
    """
    rows = _all_rows(seq_lens, rows)
    Re = A_emb.shape[1]
    out = np.zeros((len(rows), Re), dtype=A_emb.dtype)
    ids = np.asarray(input_ids, dtype=np.int64)
    for r, pos, toks in _rows_by_request(seq_lens, rows):
        a = int(req_slots[r])
        rho = min(int(lora_ranks[a]), Re)
        if rho <= 0:
            continue
        for p, t in zip(pos, toks):
            v = int(ids[t])
            if 0 <= v < vocab_size:
                out[p, :rho] = A_emb[a, :rho, v]
    return out
