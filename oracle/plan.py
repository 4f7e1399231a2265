"""Plan oracle: the chunked SGMV batch planner, written naively in pure Python.

Test infrastructure only (see the package docstring).  Every output is an
integer list and must be matched bit for bit by the native planner.

Follows the ``chunked_backend.py`` page (class ``ChunkedSgmvLoRABackend``):

* chunk size          -- ``_determine_chunk_size`` / ``_determine_chunk_size_for_tokens``
                         and the module constant ``MIN_CHUNK_SIZE``;
* gather permutation  -- ``_get_permutation`` (tokens take their request's
                         adapter slot; a stable ascending sort by slot);
* segments            -- ``_get_segments_info`` (runs of equal slots in the
                         sorted order, each cut into pieces of ``chunk`` tokens
                         with the remainder last; CSR boundaries);
* per-request routing -- ``_build_req_seg_indptr``;
* graph padding       -- the CUDA-graph branch of ``prepare_lora_batch``
                         (unused segment slots get adapter 0 and zero length);
* lm_head plans       -- ``_prepare_lm_head_batch_info`` / ``_build_lm_head_batch_info``
                         (identity permutation; segments from the page's
                         unprinted ``merge_and_chunk_segments``, read plainly:
                         see ``merge_and_chunk``).

Readings where the page is silent: in decode mode every request carries one
token; requests of length zero contribute no tokens; ``chunk_override > 0``
replaces the heuristic (needed to reproduce the page's chunk-3 example).
"""

MIN_CHUNK_SIZE = 16


def chunk_size_for_tokens(num_tokens, max_chunk_size):
    """Chunk size for a batch of ``num_tokens`` tokens.

    ``_determine_chunk_size_for_tokens``: a server cap at or below the
    minimum chunk gives the minimum; otherwise 128 for at least 256 tokens,
    32 for at least 64, else 16, never above the cap.
    """
    if max_chunk_size <= MIN_CHUNK_SIZE:
        return MIN_CHUNK_SIZE
    if num_tokens >= 256:
        wanted = 128
    elif num_tokens >= 64:
        wanted = 32
    else:
        wanted = 16
    return min(max_chunk_size, wanted)


def token_slots(seq_lens, req_slots):
    """Adapter slot of every token, requests laid out one after another.

    ``_get_permutation``: each request's slot is repeated once per token of
    that request (``repeat_interleave``), so token order is request-major.
    """
    rows = []
    for length, slot in zip(seq_lens, req_slots):
        for _ in range(length):
            rows.append(slot)
    return rows


def gather_permutation(rows):
    """Stable ascending sort of token indices by slot.

    ``_get_permutation`` sorts with ``stable=True``; sorting the pairs
    (slot, token index) lexicographically gives the same order, because the
    token index breaks ties in original order.
    Returns (permutation, slots in sorted order).
    """
    pairs = sorted((slot, t) for t, slot in enumerate(rows))
    perm = [t for _, t in pairs]
    sorted_slots = [slot for slot, _ in pairs]
    return perm, sorted_slots


def segments(sorted_slots, chunk):
    """Cut each run of equal slots into segments of at most ``chunk`` tokens.

    ``_get_segments_info``: for a run of ``n`` tokens, ``ceil(n / chunk)``
    segments -- all but the last exactly ``chunk`` long, the last holding the
    remainder.  Returns (per-segment slot, CSR boundaries starting at 0).
    """
    seg_slots = []
    seg_lens = []
    i = 0
    n = len(sorted_slots)
    while i < n:
        j = i
        while j < n and sorted_slots[j] == sorted_slots[i]:
            j += 1
        run = j - i
        pieces = (run + chunk - 1) // chunk
        for q in range(pieces):
            seg_slots.append(sorted_slots[i])
            seg_lens.append(chunk if q < pieces - 1 else run - (pieces - 1) * chunk)
        i = j
    indptr = [0]
    for length in seg_lens:
        indptr.append(indptr[-1] + length)
    return seg_slots, indptr


def request_indptr(seq_lens):
    """Per-request token boundaries ``[0, cumsum(lens)]`` (``_build_req_seg_indptr``).

    In decode mode every length is one, which gives ``0..bs`` as on the page.
    """
    out = [0]
    for length in seq_lens:
        out.append(out[-1] + length)
    return out


def plan(seq_lens, req_slots, is_decode, max_chunk_size, chunk_override=0,
         capacity=None):
    """Full batch plan, as ``prepare_lora_batch`` assembles it.

    ``seq_lens`` may be None in decode mode (one token per request).  The
    chunk heuristic sees the batch size in decode mode and the total token
    count in extend mode (``_determine_chunk_size``).  If ``capacity`` is
    larger than the number of segments, the arrays are padded the way the
    graph branch pads them: slot 0 and boundaries repeating the last value.
    """
    bs = len(req_slots)
    if seq_lens is None:
        if not is_decode:
            raise ValueError("extend mode needs sequence lengths")
        seq_lens = [1] * bs
    if len(seq_lens) != bs:
        raise ValueError("one length per request")
    if is_decode and any(length != 1 for length in seq_lens):
        raise ValueError("decode mode carries one token per request")
    if any(length < 0 for length in seq_lens):
        raise ValueError("negative length")
    num_tokens = sum(seq_lens)
    if chunk_override > 0:
        chunk = chunk_override
    else:
        chunk = chunk_size_for_tokens(bs if is_decode else num_tokens, max_chunk_size)
    rows = token_slots(seq_lens, req_slots)
    perm, sorted_slots = gather_permutation(rows)
    seg_slots, indptr = segments(sorted_slots, chunk)
    num_segments = len(seg_slots)
    if capacity is not None:
        if capacity < num_segments:
            raise ValueError("segment capacity too small")
        seg_slots = seg_slots + [0] * (capacity - num_segments)
        indptr = indptr + [indptr[-1]] * (capacity - num_segments)
    return {
        "permutation": perm,
        "sorted_slots": sorted_slots,
        "seg_indptr": indptr,
        "seg_slots": seg_slots,
        "req_seg_indptr": request_indptr(seq_lens),
        "num_segments": num_segments,
        "chunk_size": chunk,
        "num_tokens": num_tokens,
    }


# ----------------------------------------------------------- lm_head plans

def merge_and_chunk(req_slots, lens, chunk):
    """Segments of the pruned lm_head tokens, which stay in original order.

    ``_prepare_lm_head_batch_info`` (``chunked_backend.py`` page) builds them
    with ``merge_and_chunk_segments(weight_indices, pruned_lens, chunk)``, a
    helper the page imports but does not print.  Plain reading, taken here:
    requests with no pruned token carry nothing and are dropped; consecutive
    requests of one slot are merged into a run; each run is cut into pieces of
    ``chunk`` tokens, the remainder last.  Returns (per-segment slot,
    per-segment length).
    """
    runs = []
    for slot, n in zip(req_slots, lens):
        if n < 0:
            raise ValueError("negative length")
        if n == 0:
            continue
        if runs and runs[-1][0] == slot:
            runs[-1][1] += n
        else:
            runs.append([slot, n])
    seg_slots, seg_lens = [], []
    for slot, n in runs:
        pieces = (n + chunk - 1) // chunk
        for q in range(pieces):
            seg_slots.append(slot)
            seg_lens.append(chunk if q < pieces - 1 else n - (pieces - 1) * chunk)
    return seg_slots, seg_lens


def lm_head_plan(pruned_lens, req_slots, max_chunk_size, chunk_override=0, capacity=None):
    """Plan of the pruned lm_head pass (``_prepare_lm_head_batch_info`` and
    ``_build_lm_head_batch_info``): the chunk from the token-count rule over
    the pruned total, segments from ``merge_and_chunk``, CSR boundaries from
    their lengths, and the identity permutation (the pruned tokens are in
    original order).  Per-pass plans for logprob chunking are the same plan
    over the requests of one pass.  ``capacity`` pads as in ``plan``."""
    if len(pruned_lens) != len(req_slots):
        raise ValueError("one length per request")
    total = sum(pruned_lens)
    chunk = chunk_override if chunk_override > 0 else chunk_size_for_tokens(total, max_chunk_size)
    seg_slots, seg_lens = merge_and_chunk(req_slots, pruned_lens, chunk)
    indptr = [0]
    for length in seg_lens:
        indptr.append(indptr[-1] + length)
    num_segments = len(seg_slots)
    if capacity is not None:
        if capacity < num_segments:
            raise ValueError("segment capacity too small")
        seg_slots = seg_slots + [0] * (capacity - num_segments)
        indptr = indptr + [indptr[-1]] * (capacity - num_segments)
    return {
        "permutation": list(range(total)),
        "seg_indptr": indptr,
        "seg_slots": seg_slots,
        "num_segments": num_segments,
        "chunk_size": chunk,
        "num_tokens": total,
    }

