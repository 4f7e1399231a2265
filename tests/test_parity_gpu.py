"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance per output element: |gpu - oracle| <= 1e-2 + 1e-2 * |oracle| for
bf16 inputs with fp32 accumulation; plan arrays and the embedding gather are
bit-exact.  Large workloads are checked on sampled rows (segment boundaries,
first/last tokens and a seeded random sample), computed one by one by the
oracle, in the launch configuration the benchmark times.
"""

import ctypes
import zlib

import numpy as np
import pytest
import torch

from oracle import lora as ol
from oracle import moe as om
from oracle import plan as op
from synth import Batch, Projection, draw_batch, draw_embedding, draw_projection, to_f64

pytestmark = pytest.mark.gpu

ATOL = RTOL = 1e-2
COUNTER_BYTES = 65536   # workspace counter region (and the fused call's status word)


def _sgg():
    import segmented_gather_gemm_amd as sgg
    return sgg


DEV = torch.device("cuda:0")


def assert_close(got, want, what):
    got = to_f64(got) if isinstance(got, torch.Tensor) else got
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    bad = err > ATOL + RTOL * np.abs(want)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, "
                           f"max abs err {err.max():.4g}")
    return float(err.max())


def check_plan(info, b, max_chunk, override=0):
    ref = op.plan(None if b.is_decode else b.seq_lens, b.req_slots, b.is_decode, max_chunk,
                  override)
    n = info.num_segments
    assert info.max_len == ref["chunk_size"]
    assert n == ref["num_segments"]
    assert info.permutation.cpu().tolist() == ref["permutation"]
    assert info.seg_indptr[:n + 1].cpu().tolist() == ref["seg_indptr"]
    assert info.weight_indices[:n].cpu().tolist() == ref["seg_slots"]
    assert info.req_seg_indptr.cpu().tolist() == ref["req_seg_indptr"]
    check_work_segments(info, ref)
    return ref


def _work_segment_tokens():
    import os
    import re
    hdr = os.path.join(os.path.dirname(__file__), "..", "include", "sgg_lora.h")
    return int(re.search(r"#define SGG_WORK_SEGMENT_TOKENS (\d+)", open(hdr).read()).group(1))


def check_work_segments(info, ref):
    """The kernels' work segments: runs of the plan's segments of one slot,
    merged greedily while within max(chunk, SGG_WORK_SEGMENT_TOKENS) tokens
    (a coarser partition of the same sorted positions)."""
    n = info.num_work_segments
    wind = info.work_indptr[:n + 1].cpu().tolist()
    wsl = info.work_slots[:n].cpu().tolist()
    ind, sl = ref["seg_indptr"], ref["seg_slots"]
    limit = max(ref["chunk_size"], _work_segment_tokens())
    assert wind[0] == 0 and wind[-1] == ind[-1]
    pos = {v: i for i, v in enumerate(ind)}
    assert all(v in pos for v in wind)
    for w in range(n):
        lo, hi = wind[w], wind[w + 1]
        i0, i1 = pos[lo], pos[hi]
        assert i1 > i0 and all(sl[i] == wsl[w] for i in range(i0, i1))
        assert hi - lo <= limit
        if i1 < len(sl):   # greedy: the next segment differs in slot or would not fit
            assert sl[i1] != wsl[w] or ind[i1 + 1] - lo > limit


def sample_rows(ref, s, n_random=768, seed=0):
    """Tokens at every segment boundary, first/last, plus a seeded random sample."""
    perm = ref["permutation"]
    ind = ref["seg_indptr"]
    rows = {0, s - 1}
    for i in range(ref["num_segments"]):
        rows.add(perm[ind[i]])
        rows.add(perm[ind[i + 1] - 1])
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, s, size=min(n_random, s)).tolist())
    return np.array(sorted(rows), dtype=np.int64)


class fused_stacked:
    """Context: lora_qkv in its one-launch form (lora_set_option
    "fused_stacked" = 1) inside, the default two-launch form after."""

    def __enter__(self):
        self.old = _sgg().lora_set_option("fused_stacked", 1)

    def __exit__(self, *exc):
        _sgg().lora_set_option("fused_stacked", self.old)


def stacked_both_forms(x, A, Bw, info, offs, wide, base, ws):
    """lora_qkv in its default two-launch form and in its one-launch form;
    returns both results (the one-launch form twice, asserted identical)."""
    sgg = _sgg()
    y = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
    with fused_stacked():
        yf = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
        yf2 = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(yf, yf2)
    return y, yf


def own_plan(info):
    """A copy of a plan whose device arrays belong to it alone (the backend's
    ring keeps 8 live plans)."""
    import dataclasses
    return dataclasses.replace(info, **{
        f.name: getattr(info, f.name).clone() for f in dataclasses.fields(info)
        if isinstance(getattr(info, f.name), torch.Tensor)})


def backend(b, max_chunk=None):
    return _sgg().ChunkedSgmvLoRA(b.num_loras, max_chunk or b.max_chunk_size, DEV)


def plan_on(be, b, override=0):
    return be.prepare_lora_batch(None if b.is_decode else b.seq_lens, b.req_slots,
                                 b.lora_ranks, b.scalings, is_decode=b.is_decode,
                                 chunk_size_override=override)


def run_forward(be, proj, x, A, Bw, base):
    """The page's call for the projection: plain (c=1) or stacked (c>1)."""
    offs = proj.slice_offsets
    if proj.num_slices == 1:
        h = be.run_lora_a_sgemm(x, A)
        return h, be.run_lora_b_sgemm(h, Bw, offs, base)
    h = be.run_lora_a_sgemm(x, A, stack_num=proj.num_slices)
    if proj.num_slices == 3:
        y = be.run_qkv_lora(x, A, Bw, offs, proj.max_slice, base)
    else:
        y = be.run_gate_up_lora(x, A, Bw, offs, base)
    return h, y


def oracle_forward(t, b, proj, rows=None):
    x, A, Bw = to_f64(t["x"]), to_f64(t["A"]), to_f64(t["B"])
    base = to_f64(t["base"] if rows is None else t["base"][torch.as_tensor(rows)])
    h = ol.shrink(x, A, b.seq_lens, b.req_slots, b.lora_ranks, proj.num_slices, rows)
    y = ol.expand(h, Bw, base, b.seq_lens, b.req_slots, b.lora_ranks, b.scalings,
                  proj.slice_offsets, rows)
    return h, y


# ------------------------------------------------------------- workloads

def test_tiny_full():
    b = draw_batch("tiny")
    proj = b.projections[0]
    t = draw_projection(b, proj)
    be = backend(b)
    info = plan_on(be, b)
    check_plan(info, b, b.max_chunk_size)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    h, y = run_forward(be, proj, x, A, Bw, base.clone())
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "tiny h")
    assert_close(y, want_y, "tiny y")


def test_decode_full():
    b = draw_batch("decode")
    proj = b.projections[0]
    t = draw_projection(b, proj)
    be = backend(b)
    info = plan_on(be, b)
    check_plan(info, b, b.max_chunk_size)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    h, y = run_forward(be, proj, x, A, Bw, base.clone())
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "decode h")
    assert_close(y, want_y, "decode y")
    # same call again: deterministic, and the split-K workspace was left clean
    h2, y2 = run_forward(be, proj, x, A, Bw, base.clone())
    assert torch.equal(h2, h) and torch.equal(y2, y)


@pytest.mark.parametrize("case", [
    # (seed, tokens, slots, c, R, K): decode-like batches whose shrink splits K
    (61, 256, 8, 3, 16, 4096),
    (62, 40, 3, 3, 16, 2048),
    (63, 64, 4, 2, 32, 4096),
    (64, 96, 16, 1, 64, 4096),
    (65, 24, 2, 4, 16, 1024),
    (66, 64, 4, 1, 16, 14336),
    (67, 48, 3, 2, 32, 10240),
    (68, 20, 2, 3, 16, 8192),
])
def test_stacked_call_matches_separate_calls(case):
    """lora_qkv on small batches (split K: the expand sums the shrink's
    partials itself) gives the same bits as lora_shrink (whose last arriving
    workgroup sums them) followed by lora_expand, call after call, and matches
    the oracle; its one-launch form matches the oracle and repeats bit for
    bit; the workspace counter region is left at zero."""
    sgg = _sgg()
    seed, s, L, c, R, K = case
    rng = np.random.default_rng(seed)
    slots = rng.integers(0, L, size=s).tolist()
    width = [4096 if k == 0 else 1024 for k in range(c)] if K == 4096 else [512] * c
    offs = np.concatenate([[0], np.cumsum(width)]).tolist()
    b, proj, t = _small_case(seed, [1] * s, slots, L, [R] * L,
                             rng.uniform(0.5, 2.0, size=L).tolist(), K, offs, R)
    be = backend(b)
    info = plan_on(be, b)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    h = sgg.lora_shrink(x, A, info, c, workspace=ws)
    y_sep = sgg.lora_expand(h, Bw, info, offs, max(width), base.clone())
    _, want_y = oracle_forward(t, b, proj)
    assert_close(y_sep, want_y, f"case {seed} separate")
    for rep in range(3):
        y = sgg.lora_qkv(x, A, Bw, info, offs, max(width), base.clone(), workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y_sep), (seed, rep)
        assert not ws[:COUNTER_BYTES].any(), (seed, rep)
    _, yf = stacked_both_forms(x, A, Bw, info, offs, max(width), base, ws)
    assert_close(yf, want_y, f"case {seed} one launch")
    assert not ws[:COUNTER_BYTES].any(), seed


def _decode_case(seed, s=256, L=8, c=3, R=16, K=4096):
    rng = np.random.default_rng(seed)
    slots = rng.integers(0, L, size=s).tolist()
    width = [4096, 1024, 1024][:c] if K == 4096 else [512] * c
    offs = np.concatenate([[0], np.cumsum(width)]).tolist()
    b, proj, t = _small_case(seed, [1] * s, slots, L, [R] * L,
                             rng.uniform(0.5, 2.0, size=L).tolist(), K, offs, R)
    return b, proj, t, offs, max(width)


def test_fused_stacked_call_over_changing_plans():
    """One-launch stacked calls on decode batches whose plans change from call
    to call (segment counts 5..16, different token counts), back to back on
    one workspace: every call matches the oracle and repeats bit for bit,
    and the hand-off words and the status word end at zero."""
    sgg = _sgg()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    cases = [(71, 256, 8), (72, 100, 5), (73, 256, 16), (74, 37, 3), (75, 512, 12)]
    outs = []
    for seed, s, L in cases:
        b, proj, t, offs, wide = _decode_case(seed, s=s, L=L)
        be = backend(b)
        info = own_plan(plan_on(be, b))
        x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
        with fused_stacked():
            y = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
            y2 = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
        outs.append((b, proj, t, y, y2))
    torch.cuda.synchronize()
    for b, proj, t, y, y2 in outs:
        assert torch.equal(y, y2), b.seed
        _, want_y = oracle_forward(t, b, proj)
        assert_close(y, want_y, f"fused {b.seed}")
    assert not ws[:COUNTER_BYTES].any()


def test_fused_wait_gives_up_and_recomputes():
    """With a spin limit of 0 the one-launch call's consumers give up on a
    producer that has not published yet (the shrink tiles take microseconds;
    a limit of 0 polls once), compute their segment's partials themselves and
    set the status word: the result is still bit-identical to the one-launch
    call that waited, and the hand-off words still end at zero."""
    sgg = _sgg()
    b, proj, t, offs, wide = _decode_case(76)
    be = backend(b)
    info = plan_on(be, b)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    with fused_stacked():
        y_ref = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
        torch.cuda.synchronize()
        assert not ws[:COUNTER_BYTES].any()
        old = sgg.lora_set_option("spin_limit", 0)
        try:
            y = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
        finally:
            sgg.lora_set_option("spin_limit", old)
        torch.cuda.synchronize()
        status = int(ws[COUNTER_BYTES - 4:COUNTER_BYTES].view(torch.int32).item())
        assert status == 1, status
        assert torch.equal(y, y_ref)
        assert not ws[:COUNTER_BYTES - 4].any()
        ws.zero_()
        y = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
        torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert not ws[:COUNTER_BYTES].any()
    _, want_y = oracle_forward(t, b, proj)
    assert_close(y, want_y, "one launch after give-up")


def test_fused_timeline_leaves_results_unchanged():
    """The one-launch call's block timeline (lora_set_option "fused_trace"):
    with it on, the result is bit-identical to the call without it; every
    workgroup of the grid up to the capacity records start <= wait/work-done
    <= end, the roles split into the shrink tiles first and the expand tiles
    after them, and workgroups past the capacity write nothing."""
    sgg = _sgg()
    b, proj, t, offs, wide = _decode_case(79)
    be = backend(b)
    info = plan_on(be, b)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    cap = 1 << 14
    trace = torch.zeros(4 * (cap + 64), dtype=torch.int64, device=DEV)
    with fused_stacked():
        y_ref = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
        torch.cuda.synchronize()
        old_b = sgg.lora_set_option("fused_trace_blocks", cap)
        old_t = sgg.lora_set_option("fused_trace", trace.data_ptr())
        try:
            y = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
            torch.cuda.synchronize()
        finally:
            sgg.lora_set_option("fused_trace", old_t)
            sgg.lora_set_option("fused_trace_blocks", old_b)
    assert torch.equal(y, y_ref)
    tr = trace.view(-1, 4).cpu().numpy()
    assert not tr[cap:].any()
    used = tr[:cap][tr[:cap, 0] > 0]
    assert len(used) > 0
    roles = used[:, 3]
    assert set(roles.tolist()) <= {0, 1}
    # shrink tiles (role 0) occupy the first workgroups of the grid
    idx = np.nonzero(tr[:cap, 0] > 0)[0]
    assert (np.diff((tr[idx, 3] > 0).astype(int)) >= 0).all()
    waited = used[used[:, 1] > 0]
    assert (waited[:, 0] <= waited[:, 1]).all() and (waited[:, 1] <= waited[:, 2]).all()
    assert (used[:, 0] <= used[:, 2]).all()
    _, want_y = oracle_forward(t, b, proj)
    assert_close(y, want_y, "one launch with its timeline on")


def test_graph_keeps_its_default_workspace():
    """run_qkv_lora captured in a graph with the default workspace; then an
    eager call large enough to grow that workspace, and new allocations that
    would reuse freed memory; the replays still match the oracle, because an
    outgrown workspace is kept alive, not freed."""
    sgg = _sgg()
    from segmented_gather_gemm_amd import binding
    L, max_bs = 8, 256
    b0, proj, t, offs, wide = _decode_case(81, s=max_bs, L=L)
    x, A, Bw = (t[k].to(DEV) for k in ("x", "A", "B"))
    base0 = t["base"].to(DEV)
    base = base0.clone()
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    be.init_cuda_graph_batch_info(max_bs, 1)
    be.prepare_lora_batch(None, b0.req_slots, b0.lora_ranks, b0.scalings, is_decode=True,
                          use_cuda_graph=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        be.run_qkv_lora(x, A, Bw, offs, wide, base)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        be.run_qkv_lora(x, A, Bw, offs, wide, base)
    torch.cuda.synchronize()
    key = (DEV.type, DEV.index if DEV.index is not None else torch.cuda.current_device())
    ws_captured = binding._workspaces[key]
    # a call that needs a larger default workspace grows it (forced here: the
    # size the previous tests left it at is not known), then an eager call
    binding.default_workspace(DEV, ws_captured.numel() + 1)
    bb, pb, tb, offs_b, wide_b = _decode_case(82, s=4096, L=L, K=512)
    eb = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    plan_on(eb, bb)
    yb = eb.run_qkv_lora(tb["x"].to(DEV), tb["A"].to(DEV), tb["B"].to(DEV), offs_b, wide_b,
                         tb["base"].to(DEV))
    torch.cuda.synchronize()
    assert binding._workspaces[key].data_ptr() != ws_captured.data_ptr(), "workspace did not grow"
    _, want_b = oracle_forward(tb, bb, pb)
    assert_close(yb, want_b, "eager call after the capture")
    filler = [torch.full((1 << 20,), -1, dtype=torch.int32, device=DEV) for _ in range(8)]
    rng = np.random.default_rng(83)
    for trial in range(3):
        slots = rng.integers(0, L, size=max_bs).tolist()
        be.prepare_lora_batch(None, slots, b0.lora_ranks, b0.scalings, is_decode=True,
                              use_cuda_graph=True)
        base.copy_(base0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        b = Batch("g", 0, [1] * max_bs, slots, True, L, b0.lora_ranks, b0.scalings, 128,
                  b0.projections)
        _, want_y = oracle_forward(t, b, proj)
        assert_close(base, want_y, f"replay {trial} after the workspace grew")
    del filler


def test_fused_stacked_call_in_a_graph():
    """The one-launch stacked call captured in a graph over a capacity plan
    (trailing segments empty): replays with new plans, eager work and
    synchronisations between them, each checked against the oracle, and the
    hand-off words back at zero after every replay."""
    sgg = _sgg()
    L, R, max_bs = 8, 16, 256
    b0, proj, t, offs, wide = _decode_case(77, s=max_bs, L=L)
    x, A, Bw = (t[k].to(DEV) for k in ("x", "A", "B"))
    base0 = t["base"].to(DEV)
    base = base0.clone()
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device=DEV)
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    info = be.init_cuda_graph_batch_info(max_bs, 1)
    be.prepare_lora_batch(None, b0.req_slots, b0.lora_ranks, b0.scalings, is_decode=True,
                          use_cuda_graph=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with fused_stacked():
        with torch.cuda.stream(side):
            sgg.lora_qkv(x, A, Bw, info, offs, wide, base, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sgg.lora_qkv(x, A, Bw, info, offs, wide, base, workspace=ws)
        torch.cuda.synchronize()
    rng = np.random.default_rng(78)
    for trial in range(4):
        active = rng.integers(1, L + 1)
        slots = rng.integers(0, active, size=max_bs).tolist()
        be.prepare_lora_batch(None, slots, b0.lora_ranks, b0.scalings, is_decode=True,
                              use_cuda_graph=True)
        base.copy_(base0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert not ws[:COUNTER_BYTES].any(), trial
        b = Batch("g", 0, [1] * max_bs, slots, True, L, b0.lora_ranks, b0.scalings, 128,
                  b0.projections)
        _, want_y = oracle_forward(t, b, proj)
        assert_close(base, want_y, f"fused graph replay {trial}")
        torch.mm(torch.randn(64, 64, device=DEV), torch.randn(64, 64, device=DEV))


@pytest.fixture(scope="module")
def prefill_data():
    b = draw_batch("prefill")
    proj = b.projections[0]
    t = draw_projection(b, proj)
    dev = {k: t[k].to(DEV) for k in ("x", "A", "B", "base")}
    return b, proj, t, dev


@pytest.mark.parametrize("max_chunk", [16, 32, 64, 128])
def test_prefill_sampled(prefill_data, max_chunk):
    b, proj, t, dev = prefill_data
    be = backend(b, max_chunk)
    info = plan_on(be, b)
    ref = check_plan(info, b, max_chunk)
    rows = sample_rows(ref, b.num_tokens, seed=max_chunk)
    h, y = run_forward(be, proj, dev["x"], dev["A"], dev["B"], dev["base"].clone())
    want_h, want_y = oracle_forward(t, b, proj, rows)
    rows_t = torch.as_tensor(rows, device=DEV)
    assert_close(h.index_select(0, rows_t), want_h, f"prefill/{max_chunk} h")
    assert_close(y.index_select(0, rows_t), want_y, f"prefill/{max_chunk} y")
    check_every_row_fp32(b, proj, dev, h, y)


def test_prefill_segment_pair_tiles(prefill_data):
    """The shrink's segment-pair tiles (lora_set_option "shrink_pair_tiles"
    = 1: 256-token tiles over pairs of consecutive same-slot work segments,
    K in two ranges) on the prefill batch: sampled rows against the oracle,
    every row against float32 products, and the stacked call against the
    separate calls bit for bit (both sum the two K ranges in split order)."""
    sgg = _sgg()
    b, proj, t, dev = prefill_data
    old = sgg.lora_set_option("shrink_pair_tiles", 1)
    try:
        be = backend(b, 128)
        info = plan_on(be, b)
        ref = check_plan(info, b, 128)
        rows = sample_rows(ref, b.num_tokens, seed=5)
        h, y = run_forward(be, proj, dev["x"], dev["A"], dev["B"], dev["base"].clone())
        ws = torch.zeros(256 << 20, dtype=torch.uint8, device=DEV)
        h_sep = sgg.lora_shrink(dev["x"], dev["A"], info, proj.num_slices, workspace=ws)
        y_sep = sgg.lora_expand(h_sep, dev["B"], info, proj.slice_offsets, proj.max_slice,
                                dev["base"].clone())
        torch.cuda.synchronize()
    finally:
        sgg.lora_set_option("shrink_pair_tiles", old)
    assert torch.equal(y, y_sep)
    want_h, want_y = oracle_forward(t, b, proj, rows)
    rows_t = torch.as_tensor(rows, device=DEV)
    assert_close(h.index_select(0, rows_t), want_h, "prefill pair tiles h")
    assert_close(y.index_select(0, rows_t), want_y, "prefill pair tiles y")
    check_every_row_fp32(b, proj, dev, h, y)


def check_every_row_fp32(b, proj, dev, h, y):
    """Every row of a full-size result against plain float32 torch products on
    the GPU, adapter by adapter with tokens taken from the requests (no plan
    array): h against x A^T, and y against base + sigma * h B^T computed from
    the kernel's own h, so the expand is checked on every row independently of
    the shrink's rounding.  Same tolerance as the oracle comparisons."""
    c, offs = proj.num_slices, proj.slice_offsets
    R = dev["B"].shape[2]
    tok_slot = np.repeat(np.asarray(b.req_slots), b.seq_lens)
    base = dev["base"]
    for a in np.unique(tok_slot).tolist():
        rows = torch.as_tensor(np.nonzero(tok_slot == a)[0], device=DEV)
        rho = min(int(b.lora_ranks[a]), R)
        xa = dev["x"].index_select(0, rows).float()
        ha = h.index_select(0, rows).float()
        want_h = torch.zeros_like(ha)
        want_y = base.index_select(0, rows).float()
        for k in range(c):
            if rho == 0:
                break
            Ak = dev["A"][a, k * R:k * R + rho].float()
            want_h[:, k * R:k * R + rho] = xa @ Ak.t()
            Bk = dev["B"][a, offs[k]:offs[k + 1], :rho].float()
            want_y[:, offs[k]:offs[k + 1]] += float(b.scalings[a]) * (
                ha[:, k * R:k * R + rho] @ Bk.t())
        for got, want, what in ((ha, want_h, "h"), (y.index_select(0, rows).float(), want_y, "y")):
            bad = (got - want).abs() > ATOL + RTOL * want.abs()
            assert torch.isfinite(got).all(), f"slot {a} {what}: non-finite"
            assert not bad.any(), f"slot {a} {what}: {int(bad.sum())} outside tolerance"


def test_prefill_reduced_full():
    """A smaller prefill-shaped batch compared on every output element."""
    rng = np.random.default_rng(77)
    lens = rng.integers(64, 300, size=6).tolist()
    slots = rng.integers(0, 4, size=6).tolist()
    b = Batch("prefill_small", 4242, lens, slots, False, 4, [64] * 4, [1.0] * 4, 128,
              [Projection("gate_up", 4096, [0, 1024, 2048], 64)])
    proj = b.projections[0]
    t = draw_projection(b, proj)
    be = backend(b)
    info = plan_on(be, b)
    check_plan(info, b, 128)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    h, y = run_forward(be, proj, x, A, Bw, base.clone())
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "prefill-small h")
    assert_close(y, want_y, "prefill-small y")


@pytest.mark.parametrize("which", [0, 1])
def test_skewed_full(which):
    b = draw_batch("skewed")
    proj = b.projections[which]
    t = draw_projection(b, proj, proj_index=which)
    assert torch.isnan(t["A"].float()).any() and torch.isnan(t["B"].float()).any()
    be = backend(b)
    info = plan_on(be, b)
    check_plan(info, b, b.max_chunk_size)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    h, y = run_forward(be, proj, x, A, Bw, base.clone())
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, f"skewed/{proj.name} h")
    assert_close(y, want_y, f"skewed/{proj.name} y")


@pytest.mark.parametrize("layer", [0, 31])
def test_full_sweep_layers(layer):
    b = draw_batch("full")
    be = backend(b)
    info = plan_on(be, b)
    ref = check_plan(info, b, b.max_chunk_size)
    rows = sample_rows(ref, b.num_tokens, n_random=512, seed=layer)
    rows_t = torch.as_tensor(rows, device=DEV)
    for pi, proj in enumerate(b.projections):
        t = draw_projection(b, proj, layer=layer, proj_index=pi)
        x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
        h, y = run_forward(be, proj, x, A, Bw, base.clone())
        want_h, want_y = oracle_forward(t, b, proj, rows)
        assert_close(h.index_select(0, rows_t), want_h, f"full/L{layer}/{proj.name} h")
        assert_close(y.index_select(0, rows_t), want_y, f"full/L{layer}/{proj.name} y")


def test_full_embedding_bit_exact():
    b = draw_batch("full")
    ids, A_emb = draw_embedding(b)
    be = backend(b)
    plan_on(be, b)
    e = be.run_lora_a_embedding(ids.to(DEV), A_emb.to(DEV), b.vocab_size)
    want = ol.embedding_a(ids.numpy(), to_f64(A_emb), b.seq_lens, b.req_slots, b.lora_ranks,
                          b.vocab_size)
    assert np.array_equal(to_f64(e), want)


# ---------------------------------------------------- invariances and edges

def _small_case(seed, lens, slots, L, ranks, scal, K, offs, R, nan_pad=False):
    b = Batch("case", seed, list(lens), list(slots), False, L, list(ranks), list(scal), 128,
              [Projection("p", K, list(offs), R)], nan_padding=nan_pad)
    return b, b.projections[0], draw_projection(b, b.projections[0])


def _gpu_forward(b, proj, t, override=0, max_chunk=128):
    be = backend(b, max_chunk)
    info = plan_on(be, b, override)
    check_plan(info, b, max_chunk, override)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    h, y = run_forward(be, proj, x, A, Bw, base.clone())
    torch.cuda.synchronize()
    return h, y


class shrink_valu:
    """Context: the shrink's VALU form of short tiles (lora_set_option
    "shrink_valu" = 1) inside, the default MFMA form after."""

    def __enter__(self):
        self.old = _sgg().lora_set_option("shrink_valu", 1)

    def __exit__(self, *exc):
        _sgg().lora_set_option("shrink_valu", self.old)


def _valu_cases():
    rng = np.random.default_rng(41)
    one = ("one_token_segments", [1] * 256, rng.integers(0, 128, 256).tolist(), 128,
           rng.choice([16, 8, 12, 0], 128).tolist(), 4096, [0, 512, 640, 768], 16, 0)
    mixed = ("mixed", [1] * 40 + [3, 2, 4, 5, 37, 70], rng.integers(0, 32, 46).tolist(), 32,
             [32] * 32, 1024, [0, 384], 32, 0)
    ragged = ("ragged_k_chunk_1", [2, 1, 3, 9, 4, 1, 6], [0, 1, 2, 1, 0, 3, 2], 4,
              [8, 5, 8, 3], 1000, [0, 100, 200], 8, 1)
    return [one, mixed, ragged]


@pytest.mark.parametrize("case", _valu_cases(), ids=lambda c: c[0])
def test_shrink_valu_short_tiles(case):
    """The shrink's VALU form (16-token tiles; those with at most 4 tokens
    summed on the VALU with cross-lane reductions, the rest on MFMA): h and y
    match the oracle on one-token segments of a many-adapter decode batch, a
    mix of short and long segments, and a ragged K with chunk size 1; the
    stacked call in this form matches the separate calls bit for bit."""
    name, lens, slots, L, ranks, K, offs, R, override = case
    sgg = _sgg()
    scal = np.random.default_rng(42).uniform(0.5, 2.0, L).tolist()
    b, proj, t = _small_case(43, lens, slots, L, ranks, scal, K, offs, R)
    with shrink_valu():
        h, y = _gpu_forward(b, proj, t, override)
        want_h, want_y = oracle_forward(t, b, proj)
        assert_close(h, want_h, f"{name} h (VALU tiles)")
        assert_close(y, want_y, f"{name} y (VALU tiles)")
        be = backend(b)
        info = own_plan(plan_on(be, b, override))
        x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
        ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
        wide = int(max(np.diff(offs)))
        c = proj.num_slices
        y_st = sgg.lora_qkv(x, A, Bw, info, offs, wide, base.clone(), workspace=ws)
        h_sep = sgg.lora_shrink(x, A, info, c, workspace=ws)
        y_sep = sgg.lora_expand(h_sep, Bw, info, offs, wide, base.clone())
        torch.cuda.synchronize()
    assert torch.equal(y_st, y_sep), name
    assert_close(y_st, want_y, f"{name} stacked (VALU tiles)")


def _random_batch_case(seed):
    """A seeded random batch: decode or extend, 1-12 adapters with ranks
    anywhere in [0, R], 1-3 slices (gate_up halves equal), K a multiple of 8,
    chunk cap and override drawn too."""
    rng = np.random.default_rng(seed)
    decode = rng.random() < 0.3
    bs = int(rng.integers(1, 41))
    lens = [1] * bs if decode else rng.integers(0, 71, size=bs).tolist()
    L = int(rng.integers(1, 13))
    slots = rng.integers(0, L, size=bs).tolist()
    R = int(rng.choice([8, 16, 32, 64]))
    ranks = rng.integers(0, R + 1, size=L).tolist()
    scal = rng.uniform(-2.0, 2.0, size=L).tolist()
    c = int(rng.integers(1, 4))
    K = 8 * int(rng.integers(1, 257))
    if c == 2:
        w = int(rng.integers(1, 200))
        widths = [w, w]
    else:
        widths = rng.integers(1, 300, size=c).tolist()
    offs = np.concatenate([[0], np.cumsum(widths)]).astype(int).tolist()
    cap = int(rng.choice([16, 32, 64, 128]))
    override = int(rng.choice([0, 0, 0, 1, 5, 16]))
    b = Batch("rand", seed, lens, slots, decode, L, ranks, scal, cap, [Projection("p", K, offs, R)])
    return b, b.projections[0], draw_projection(b, b.projections[0]), cap, override


@pytest.mark.parametrize("seed", range(24))
def test_random_batches_match_oracle(seed):
    """Seeded random batches (shapes, ranks, slices, chunk caps, overrides):
    the page's calls against the oracle, and the stacked call against the
    separate calls bit for bit."""
    sgg = _sgg()
    b, proj, t, cap, override = _random_batch_case(9000 + seed)
    be = backend(b, cap)
    info = own_plan(plan_on(be, b, override))
    check_plan(info, b, cap, override)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    offs, c = proj.slice_offsets, proj.num_slices
    h = sgg.lora_shrink(x, A, info, c, workspace=ws)
    y_sep = sgg.lora_expand(h, Bw, info, offs, proj.max_slice, base.clone())
    y_st = sgg.lora_qkv(x, A, Bw, info, offs, proj.max_slice, base.clone(), workspace=ws)
    torch.cuda.synchronize()
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, f"random {seed} h")
    assert_close(y_sep, want_y, f"random {seed} y")
    assert torch.equal(y_st, y_sep), f"random {seed}: stacked call differs from separate calls"


@pytest.mark.parametrize("override", [1, 3, 16, 32, 64, 128, 0])
def test_chunk_size_invariance(override):
    b, proj, t = _small_case(31, [5, 40, 1, 77, 130, 9], [2, 0, 2, 1, 0, 3], 4, [16] * 4,
                             [1.0, 0.5, 2.0, 1.5], 512, [0, 256, 320, 384], 16)
    h, y = _gpu_forward(b, proj, t, override)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, f"chunk {override} h")
    assert_close(y, want_y, f"chunk {override} y")


def test_large_batch_ragged_k():
    """A batch large enough for the whole-K GEMM shrink tiles, with K not a
    multiple of 64 (17 K steps, the last partly past K), NaN rank padding
    and mixed ranks; every element against the oracle."""
    rng = np.random.default_rng(91)
    lens = rng.integers(40, 300, size=48).tolist()
    slots = rng.integers(0, 40, size=48).tolist()
    ranks = [(8, 16, 24, 32)[a % 4] for a in range(40)]
    b, proj, t = _small_case(91, lens, slots, 40, ranks, rng.uniform(0.5, 2, 40).tolist(), 1064,
                             [0, 768, 1536], 32, nan_pad=True)
    h, y = _gpu_forward(b, proj, t)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "ragged-K GEMM h")
    assert_close(y, want_y, "ragged-K GEMM y")


def test_long_segment_gemm_ragged_k():
    """Long segments (mean work segment >= 96 tokens, chunk 128) and c*R =
    128 over about 33k tokens take the 128 x 128 GEMM shrink tiles with one
    register set, whose ragged-K tail (K = 1064: 17 K steps, the last partly
    past K) is zeroed at the load; NaN rank padding and mixed ranks; every
    element against the oracle."""
    rng = np.random.default_rng(93)
    lens = rng.integers(900, 1200, size=32).tolist()
    slots = rng.integers(0, 8, size=32).tolist()
    ranks = [64, 48, 64, 32, 64, 64, 16, 64]
    b, proj, t = _small_case(93, lens, slots, 8, ranks, rng.uniform(0.5, 2, 8).tolist(), 1064,
                             [0, 256, 512], 64, nan_pad=True)
    assert b.num_tokens > 32768
    h, y = _gpu_forward(b, proj, t)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "long-segment ragged-K GEMM h")
    assert_close(y, want_y, "long-segment ragged-K GEMM y")


@pytest.mark.parametrize("case", ["gemm", "split", "one_range"])
def test_strided_x(case):
    """x as a column view of a wider tensor (row stride K + 64): the buffer
    loads of the GEMM tiles (64 x 32 here), the decode split-K shrink and the
    one-range split-K kernel (short segments, c*R = 32) read the right rows;
    stacked and separate calls against the oracle on every element."""
    sgg = _sgg()
    rng = np.random.default_rng({"gemm": 97, "split": 98, "one_range": 99}[case])
    if case == "gemm":
        lens = rng.integers(40, 300, size=48).tolist()
        slots = rng.integers(0, 40, size=48).tolist()
        L, R, K, offs = 40, 32, 1024, [0, 768, 1536]
    elif case == "split":
        lens = [1] * 256
        slots = rng.integers(0, 8, size=256).tolist()
        L, R, K, offs = 8, 16, 2048, [0, 512, 768, 1024]
    else:
        lens = [1] * 192 + [512] * 4
        slots = rng.integers(0, 32, size=196).tolist()
        L, R, K, offs = 32, 32, 2048, [0, 1024]
    b, proj, t = _small_case(97, lens, slots, L, [R] * L, rng.uniform(0.5, 2, L).tolist(), K,
                             offs, R)
    be = backend(b)
    info = plan_on(be, b)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    wide = torch.full((x.shape[0], K + 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    wide[:, :K] = x
    xs = wide[:, :K]
    assert xs.stride(0) == K + 64
    c = len(offs) - 1
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    h = sgg.lora_shrink(xs, A, info, c, workspace=ws)
    y_sep = sgg.lora_expand(h, Bw, info, offs, max(np.diff(offs)), base.clone())
    y, yf = stacked_both_forms(xs, A, Bw, info, offs, max(np.diff(offs)), base, ws)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, f"strided x ({case}) h")
    assert_close(y_sep, want_y, f"strided x ({case}) y")
    assert_close(yf, want_y, f"strided x ({case}) one-launch y")
    assert torch.equal(y, y_sep)


@pytest.mark.parametrize("case", ["split", "one_range"])
def test_tiles_past_the_rank(case):
    """Ranks well below the padded R (NaN padding): split-K shrink tiles
    whose rank rows all lie past the slot's rank read nothing and write zero
    rows, on the K-split path (standalone last-arriver sum and the stacked
    call's partials) and on the one-range path; every element against the
    oracle, stacked and separate calls bit for bit."""
    sgg = _sgg()
    rng = np.random.default_rng({"split": 101, "one_range": 102}[case])
    if case == "split":
        lens = [1] * 96
        slots = rng.integers(0, 6, size=96).tolist()
        L, R, ranks, K, offs = 6, 64, [8, 16, 0, 64, 12, 32], 2048, [0, 512, 1024]
    else:
        lens = [1] * 2000 + [300] * 2
        slots = rng.integers(0, 40, size=2002).tolist()
        L, R, K, offs = 40, 32, 1024, [0, 768]
        ranks = [(8, 16, 0, 32, 12)[a % 5] for a in range(L)]
    b, proj, t = _small_case(101, lens, slots, L, ranks, rng.uniform(0.5, 2, L).tolist(), K,
                             offs, R, nan_pad=True)
    be = backend(b)
    info = plan_on(be, b)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    c = len(offs) - 1
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    h = sgg.lora_shrink(x, A, info, c, workspace=ws)
    y_sep = sgg.lora_expand(h, Bw, info, offs, max(np.diff(offs)), base.clone())
    y, yf = stacked_both_forms(x, A, Bw, info, offs, max(np.diff(offs)), base, ws)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, f"past-rank tiles ({case}) h")
    assert_close(y_sep, want_y, f"past-rank tiles ({case}) y")
    assert_close(yf, want_y, f"past-rank tiles ({case}) one-launch y")
    assert torch.equal(y, y_sep)
    assert not ws[:COUNTER_BYTES].any()


def test_long_k_small_grid():
    """Long K (129 K steps, the last partly past K) on a small grid, NaN rank
    padding, a rank-0 slot: the standalone shrink and the stacked call
    against the oracle on every element and against each other bit for bit;
    the workspace counters are left at zero."""
    sgg = _sgg()
    rng = np.random.default_rng(95)
    lens = rng.integers(60, 140, size=40).tolist()
    slots = rng.integers(0, 10, size=40).tolist()
    ranks = [16, 16, 8, 16, 16, 0, 16, 12, 16, 16]
    b, proj, t = _small_case(95, lens, slots, 10, ranks, rng.uniform(0.5, 2, 10).tolist(), 8232,
                             [0, 640, 1280], 16, nan_pad=True)
    be = backend(b)
    info = plan_on(be, b)
    check_plan(info, b, 128)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    h = sgg.lora_shrink(x, A, info, 2, workspace=ws)
    y_sep = sgg.lora_expand(h, Bw, info, proj.slice_offsets, proj.max_slice, base.clone())
    y, yf = stacked_both_forms(x, A, Bw, info, proj.slice_offsets, proj.max_slice, base, ws)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "long-K h")
    assert_close(y_sep, want_y, "long-K y (separate)")
    assert_close(yf, want_y, "long-K y (one launch)")
    assert torch.equal(y, y_sep)
    assert not ws[:COUNTER_BYTES].any()


LONG_K_CASES = [
    # (name, seed, K, slice offsets, R, ranks drawn from): batches of short
    # segments with c*R <= 32 and K >= 8192 take 64-token tiles over all rank
    # rows with K split (ranges of 1792), the last range ragged for K = 9000
    ("c1_R32_K14336", 61, 14336, [0, 1024], 32, [32]),
    ("c2_R16_K9000", 62, 9000, [0, 640, 1280], 16, [16, 16, 9, 0, 4]),
    # c*R = 8: a grid this small takes the decode-sized K split instead (2 ranges)
    ("c1_R8_K8192_small_grid", 63, 8192, [0, 512], 8, [8, 8, 3, 0]),
]


@pytest.mark.parametrize("case", LONG_K_CASES, ids=[c[0] for c in LONG_K_CASES])
def test_long_k_short_segments(case):
    """The long-K split-K tiles: the standalone shrink (split-K completion)
    and expand against the oracle on every element, NaN rank padding, rank-0
    and partial ranks; with two slices the stacked call bit for bit against
    the separate calls; the workspace counters left at zero."""
    sgg = _sgg()
    from segmented_gather_gemm_amd._lib import calls
    name, seed, K, offs, R, rank_pool = case
    rng = np.random.default_rng(seed)
    n_req, L = 150, 40
    lens = rng.integers(1, 31, size=n_req).tolist()
    slots = rng.integers(0, L, size=n_req).tolist()
    ranks = [int(rng.choice(rank_pool)) for _ in range(L)]
    b, proj, t = _small_case(seed, lens, slots, L, ranks, rng.uniform(0.5, 2, L).tolist(), K,
                             offs, R, nan_pad=True)
    be = backend(b)
    info = plan_on(be, b)
    check_plan(info, b, 128)
    c = len(offs) - 1
    ind, sl, nseg, hint, perm = info.kernel_segments()
    assert calls().lora_shrink_workspace_bytes(b.num_tokens, K, c, R, nseg, hint) > COUNTER_BYTES
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    h = sgg.lora_shrink(x, A, info, c, workspace=ws)
    y_sep = sgg.lora_expand(h, Bw, info, proj.slice_offsets, proj.max_slice, base.clone())
    torch.cuda.synchronize()
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, f"{name} h")
    assert_close(y_sep, want_y, f"{name} y")
    if c > 1:
        y = sgg.lora_qkv(x, A, Bw, info, proj.slice_offsets, proj.max_slice, base.clone(),
                         workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y_sep)
    assert not ws[:COUNTER_BYTES].any()


@pytest.mark.parametrize("n, ranges", [(1024, 4), (2048, 2)])
def test_decode_mid_sizes(n, ranges):
    """Decode-shaped batches of 1024 and 2048 tokens (8 adapters, stacked
    qkv, r = 16) take 16-token tiles over all 48 rank rows with K in 4 or 2
    ranges: shrink and expand against the oracle on every element, the
    stacked call bit for bit against the separate calls."""
    sgg = _sgg()
    from segmented_gather_gemm_amd._lib import calls
    rng = np.random.default_rng(1002 + n)
    b = Batch(f"decode_{n}", 1002 + n, [1] * n, rng.integers(0, 8, n).tolist(), True, 8,
              [16] * 8, [1.0] * 8, 128, [Projection("qkv", 4096, [0, 4096, 5120, 6144], 16)])
    proj = b.projections[0]
    t = draw_projection(b, proj)
    be = backend(b)
    info = plan_on(be, b)
    check_plan(info, b, 128)
    ind, sl, nseg, hint, perm = info.kernel_segments()
    need = calls().lora_shrink_workspace_bytes(n, 4096, 3, 16, nseg, hint)
    assert need == COUNTER_BYTES + ranges * n * 48 * 4
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    h = sgg.lora_shrink(x, A, info, 3, workspace=ws)
    y_sep = sgg.lora_expand(h, Bw, info, proj.slice_offsets, proj.max_slice, base.clone())
    y = sgg.lora_qkv(x, A, Bw, info, proj.slice_offsets, proj.max_slice, base.clone(),
                     workspace=ws)
    torch.cuda.synchronize()
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, f"decode {n} h")
    assert_close(y_sep, want_y, f"decode {n} y")
    assert torch.equal(y, y_sep)
    assert not ws[:COUNTER_BYTES].any()


def test_decode_16384_gemm_tiles():
    """A decode-shaped batch of 16384 tokens (8 adapters, stacked qkv, r =
    16) takes 64 x 64 GEMM tiles: sampled rows (every segment boundary plus a
    seeded sample) against the oracle, the stacked call bit for bit against
    the separate calls on every row."""
    sgg = _sgg()
    n = 16384
    rng = np.random.default_rng(1002 + n)
    b = Batch(f"decode_{n}", 1002 + n, [1] * n, rng.integers(0, 8, n).tolist(), True, 8,
              [16] * 8, [1.0] * 8, 128, [Projection("qkv", 4096, [0, 4096, 5120, 6144], 16)])
    proj = b.projections[0]
    t = draw_projection(b, proj)
    be = backend(b)
    info = plan_on(be, b)
    ref = check_plan(info, b, 128)
    rows = sample_rows(ref, n, seed=16384)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    h = sgg.lora_shrink(x, A, info, 3, workspace=ws)
    y_sep = sgg.lora_expand(h, Bw, info, proj.slice_offsets, proj.max_slice, base.clone())
    y = sgg.lora_qkv(x, A, Bw, info, proj.slice_offsets, proj.max_slice, base.clone(),
                     workspace=ws)
    torch.cuda.synchronize()
    want_h, want_y = oracle_forward(t, b, proj, rows)
    rows_t = torch.as_tensor(rows, device=DEV)
    assert_close(h.index_select(0, rows_t), want_h, "decode 16384 h")
    assert_close(y_sep.index_select(0, rows_t), want_y, "decode 16384 y")
    assert torch.equal(y, y_sep)


def test_short_segments_in_groups():
    """Many short segments (forced chunk 8) on few slots: the planner merges
    consecutive segments of one slot into work segments of up to
    max(chunk, SGG_WORK_SEGMENT_TOKENS) tokens, and the kernels run over those.
    Every element is compared with the oracle."""
    rng = np.random.default_rng(81)
    lens = rng.integers(1, 9, size=1800).tolist()
    slots = rng.integers(0, 6, size=1800).tolist()
    b, proj, t = _small_case(81, lens, slots, 6, [16, 16, 8, 16, 0, 16],
                             [1.0, 0.5, 2.0, 1.5, 1.0, 0.25], 1024, [0, 1024, 2048], 16)
    assert b.num_tokens > 8000
    h, y = _gpu_forward(b, proj, t, override=8)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "grouped h")
    assert_close(y, want_y, "grouped y")


def test_lm_head_pruned_pass():
    """The pruned lm_head pass: tokens stay in original order (identity
    permutation) and segments are runs of consecutive same-slot requests cut
    into chunks.  Plan arrays bit-exact with the oracle; shrink and expand
    over that plan against the oracle's per-token math on every element;
    then per-pass plans over three request ranges, likewise."""
    rng = np.random.default_rng(101)
    bs = 96
    slots = np.repeat(rng.integers(0, 6, size=40), rng.integers(1, 5, size=40))[:bs].tolist()
    lens = rng.choice([0, 1, 1, 1, 1, 2, 7, 40, 180], size=bs).tolist()
    ranks = [16, 8, 16, 0, 16, 12]
    b, proj, t = _small_case(101, lens, slots, 6, ranks, rng.uniform(0.5, 2, 6).tolist(), 2048,
                             [0, 5000], 16, nan_pad=True)
    be = backend(b)
    info = be.prepare_lm_head_batch(lens, slots, b.lora_ranks, b.scalings)
    ref = op.lm_head_plan(lens, slots, 128)
    n = info.num_segments
    assert n == ref["num_segments"] and info.max_len == ref["chunk_size"]
    assert info.permutation.cpu().tolist() == ref["permutation"]
    assert info.seg_indptr[:n + 1].cpu().tolist() == ref["seg_indptr"]
    assert info.weight_indices[:n].cpu().tolist() == ref["seg_slots"]
    # the kernels run over the pruned tokens sorted by slot: the work
    # permutation and segments are the chunked plan of the pruned tokens
    sref = op.plan(lens, slots, False, 128)
    assert info.work_perm.cpu().tolist() == sref["permutation"]
    check_work_segments(info, sref)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    h = be.run_lora_a_sgemm(x, A, pruned_batch_info=info)
    y = be.run_lora_b_sgemm(h, Bw, base_output=base.clone(), pruned_batch_info=info)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "lm_head h")
    assert_close(y, want_y, "lm_head y")

    cuts = [0, 30, 70, bs]
    passes = [(slots[a:z], lens[a:z]) for a, z in zip(cuts, cuts[1:])]
    infos = be.prepare_lm_head_pass_batches(passes, b.lora_ranks, b.scalings)
    cum = np.concatenate([[0], np.cumsum(lens)])
    for (wi, pl), pinfo, a, z in zip(passes, infos, cuts, cuts[1:]):
        pref = op.lm_head_plan(pl, wi, 128)
        pn = pinfo.num_segments
        assert pinfo.seg_indptr[:pn + 1].cpu().tolist() == pref["seg_indptr"]
        assert pinfo.weight_indices[:pn].cpu().tolist() == pref["seg_slots"]
        psref = op.plan(pl, wi, False, 128)
        assert pinfo.work_perm.cpu().tolist() == psref["permutation"]
        check_work_segments(pinfo, psref)
        rows = torch.arange(int(cum[a]), int(cum[z]), device=DEV)
        if rows.numel() == 0:
            continue
        hp = be.run_lora_a_sgemm(x.index_select(0, rows).contiguous(), A, pruned_batch_info=pinfo)
        assert_close(hp, want_h[int(cum[a]):int(cum[z])], f"lm_head pass {a}..{z} h")


def test_request_permutation_and_merge():
    lens, slots = [7, 3, 20, 3, 50, 1], [1, 1, 0, 2, 0, 0]
    b, proj, t = _small_case(32, lens, slots, 3, [8, 8, 8], [1.0, 2.0, 0.5], 256,
                             [0, 128, 256], 8)
    _, y = _gpu_forward(b, proj, t)
    y = to_f64(y)
    # requests in another order: permute x / base rows and compare back
    order = [4, 2, 0, 5, 1, 3]
    cum = np.concatenate([[0], np.cumsum(lens)])
    tok = np.concatenate([np.arange(cum[i], cum[i + 1]) for i in order])
    b2 = Batch("perm", b.seed, [lens[i] for i in order], [slots[i] for i in order], False, 3,
               b.lora_ranks, b.scalings, 128, b.projections)
    t2 = {"x": t["x"][tok], "A": t["A"], "B": t["B"], "base": t["base"][tok]}
    _, y2 = _gpu_forward(b2, proj, t2)
    assert_close(to_f64(y2), y[tok], "request order")
    # merge the two adjacent slot-1 requests, and the adjacent slot-0 pair
    b3 = Batch("merge", b.seed, [10, 20, 3, 51], [1, 0, 2, 0], False, 3, b.lora_ranks,
               b.scalings, 128, b.projections)
    _, y3 = _gpu_forward(b3, proj, t)
    assert_close(to_f64(y3), y, "request merge")


def test_rank_zero_and_zero_adapter_leave_base_bit_exact():
    # slot 0 is the base model (rank 0), slot 1 has an all-zero A
    b, proj, t = _small_case(33, [4, 9, 2, 30], [0, 1, 0, 2], 3, [0, 16, 16], [0.0, 1.0, 1.0],
                             256, [0, 256], 16)
    t["A"][1].zero_()
    h, y = _gpu_forward(b, proj, t)
    base = to_f64(t["base"])
    yy = to_f64(y)
    tokens_0 = np.r_[0:4, 13:15]
    tokens_1 = np.r_[4:13]
    assert np.array_equal(yy[tokens_0], base[tokens_0])
    assert np.array_equal(yy[tokens_1], base[tokens_1])
    assert (to_f64(h)[np.r_[tokens_0, tokens_1]] == 0).all()
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(y, want_y, "rank-0 y")


def test_nan_rank_padding_and_partial_ranks():
    # ranks not multiples of 8 inside a padded R of 24; NaN beyond each rank
    b, proj, t = _small_case(34, [17, 33, 2, 64], [0, 1, 2, 3], 4, [5, 24, 8, 13],
                             [1.0, 0.25, 2.0, 1.0], 136, [0, 72, 100, 124], 24, nan_pad=True)
    assert torch.isnan(t["A"].float()).any()
    h, y = _gpu_forward(b, proj, t)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "partial-rank h")
    assert_close(y, want_y, "partial-rank y")


def test_ragged_k_and_unaligned_slices():
    # K not a multiple of 32 or 128; slice widths not multiples of 4
    b, proj, t = _small_case(35, [3, 19, 40], [1, 0, 1], 2, [16, 16], [1.0, -0.5], 264,
                             [0, 37, 38, 101], 16)
    h, y = _gpu_forward(b, proj, t)
    want_h, want_y = oracle_forward(t, b, proj)
    assert_close(h, want_h, "ragged h")
    assert_close(y, want_y, "ragged y")


def test_columns_past_last_offset_untouched():
    b, proj, t = _small_case(36, [10, 5], [0, 1], 2, [16, 16], [1.0, 1.0], 256, [0, 96], 16)
    t["base"] = torch.randn(15, 160).to(torch.bfloat16)
    _, y = _gpu_forward(b, proj, t)
    assert torch.equal(y[:, 96:].cpu(), t["base"][:, 96:])


def test_out_of_range_slot_is_no_adapter():
    sgg = _sgg()
    b, proj, t = _small_case(37, [6, 10], [0, 1], 2, [16, 16], [1.0, 1.0], 256, [0, 128], 16)
    be = backend(b)
    info = plan_on(be, b)
    # slot outside [0, 2) in the segments the kernels run over: no adapter
    _, slots, n, _, _ = info.kernel_segments()
    slots[:n] = 7
    info.weight_indices[:info.num_segments] = 7
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    h = sgg.lora_shrink(x, A, info, 1)
    y = sgg.lora_expand(h, Bw, info, [0, 128], 128, base.clone())
    assert (h == 0).all()
    assert torch.equal(y, base)


def test_empty_batch():
    sgg = _sgg()
    be = sgg.ChunkedSgmvLoRA(2, 128, DEV)
    info = be.prepare_lora_batch([0, 0], [0, 1], [8, 8], [1.0, 1.0])
    assert info.num_tokens == 0 and info.num_segments == 0
    x = torch.zeros(0, 256, dtype=torch.bfloat16, device=DEV)
    A = torch.zeros(2, 8, 256, dtype=torch.bfloat16, device=DEV)
    h = be.run_lora_a_sgemm(x, A)
    assert h.shape == (0, 8)


def test_workspace_reuse_across_shapes():
    """Split-K counters must be left clean for a later call of another shape."""
    d = draw_batch("decode")
    proj = d.projections[0]
    t = draw_projection(d, proj)
    be = backend(d)
    plan_on(be, d)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    h1 = be.run_lora_a_sgemm(x, A, stack_num=3)
    # a smaller decode-like batch in between (different split and counters)
    b2, p2, t2 = _small_case(38, [1] * 40, [i % 3 for i in range(40)], 3, [16] * 3, [1.0] * 3,
                             2048, [0, 512], 16)
    h_small, _ = _gpu_forward(b2, p2, t2)
    want_small, _ = oracle_forward(t2, b2, p2)
    assert_close(h_small, want_small, "interleaved small h")
    plan_on(be, d)
    h2 = be.run_lora_a_sgemm(x, A, stack_num=3)
    assert torch.equal(h1, h2)


EMBED_CASES = [
    # (name, R, seq_lens, slots, num_loras, ranks, override): plans of at most
    # 63 segments take the position-major gather, larger ones the
    # segment-major one; both must give the oracle's bits.
    ("R8_zero_lengths", 8, [0, 5, 0, 3, 7, 0, 1], [2, 0, 1, 2, 4, 3, 0], 5, [8, 0, 3, 8, 5], 0),
    ("R24_straddles_waves", 24, [9, 4, 11, 2], [1, 0, 1, 2], 3, [24, 7, 16], 0),
    ("R128_token_over_two_waves", 128, [3, 2, 4], [0, 1, 0], 2, [128, 65], 0),
    ("63_segments", 16, [4] * 63, list(range(63)), 63, [16] * 63, 0),
    ("64_segments", 16, [4] * 64, list(range(64)), 64, [16] * 64, 0),
    ("override3_many_short", 16, [7, 5, 9, 3], [0, 1, 0, 2], 3, [16, 9, 4], 3),
]


@pytest.mark.parametrize("case", EMBED_CASES, ids=[c[0] for c in EMBED_CASES])
def test_embedding_plans(case):
    """The LoRA-A embedding gather, bit for bit against the oracle, on both
    of its forms: zero-length requests, partial and zero ranks, ranks whose
    (token, j) pairs straddle or span waves, and plans of 63 and 64
    segments."""
    sgg = _sgg()
    name, R, lens, slots, L, ranks, override = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    b = Batch(name, 0, lens, slots, False, L, ranks, [1.0] * L, 128)
    V = 300
    s = sum(lens)
    ids = torch.tensor(rng.integers(-2, V + 3, s), dtype=torch.int64)
    A_emb = torch.randn(L, R, V).to(torch.bfloat16)
    be = backend(b)
    plan_on(be, b, override)
    e = be.run_lora_a_embedding(ids.to(DEV), A_emb.to(DEV), V)
    want = ol.embedding_a(ids.numpy(), to_f64(A_emb), lens, slots, ranks, V)
    assert np.array_equal(to_f64(e), want)


def test_embedding_edges():
    sgg = _sgg()
    b = Batch("emb", 39, [3, 4, 2], [2, 0, 1], False, 3, [16, 0, 5], [1.0] * 3, 128)
    V = 500
    ids = torch.tensor([0, 499, 500, 7, -3, 250, 1, 2, 3], dtype=torch.int64)
    A_emb = torch.randn(3, 16, V).to(torch.bfloat16)
    be = backend(b)
    plan_on(be, b)
    e = be.run_lora_a_embedding(ids.to(DEV), A_emb.to(DEV), V)
    want = ol.embedding_a(ids.numpy(), to_f64(A_emb), b.seq_lens, b.req_slots, b.lora_ranks, V)
    assert np.array_equal(to_f64(e), want)
    with pytest.raises(NotImplementedError):
        be.run_lora_a_embedding(ids.to(DEV), A_emb.to(DEV), V, extra_embeddings=A_emb)
    with pytest.raises(sgg.SggError):
        sgg.lora_a_embedding(ids.to(DEV), A_emb.to(DEV), be.batch_info, V, extra_embeddings=1)


UPLOAD_EMBED_CASES = [
    # (name, lens (None: decode mode), bs, L, ranks, R): decode-shaped
    # batches of at most 3072 tokens over at most 64 slots take the one-launch
    # form (slots and ranks, clamped to [0, R], in the kernel arguments); the
    # others (more tokens or slots, longer requests) the two launches.
    ("decode256_L8", None, 256, 8, [16, 8, 0, 16, 4, 16, 1, 16], 16),
    ("decode256_negative_rank", None, 256, 8, [-3, 8, 0, 16, 4, 16, 1, 16], 16),
    ("decode385_mixed_ranks", None, 385, 8, "mixed", 16),
    ("rank_above_16_bits", None, 64, 4, [70000, 8, 16, 0], 16),
    ("unit_lens_extend", "ones", 200, 5, [16, 0, 9, 16, 3], 16),
    ("decode1_rank_above_R", None, 1, 2, [40, 3], 32),
    ("decode3072_L64", None, 3072, 64, "mixed", 16),
    ("decode3073_two_launches", None, 3073, 8, "mixed", 16),
    ("decode100_L65_two_launches", None, 100, 65, "mixed", 16),
    ("extend_two_launches", "random", 40, 6, [16, 8, 0, 16, 2, 11], 16),
]


@pytest.mark.parametrize("case", UPLOAD_EMBED_CASES, ids=[c[0] for c in UPLOAD_EMBED_CASES])
def test_plan_upload_embedding(case):
    """prepare_lora_batch_with_embedding: the same device plan as
    prepare_lora_batch (every region, bit for bit) and the same embedding
    rows as the oracle, in the one-launch form and in the two-launch one."""
    name, lens_kind, bs, L, ranks, R = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if ranks == "mixed":
        ranks = [int(v) for v in rng.choice([0, 4, 8, 16], L)]
    slots = [int(v) for v in rng.integers(0, L, bs)]
    if lens_kind is None:
        lens, is_decode = [1] * bs, True
    elif lens_kind == "ones":
        lens, is_decode = [1] * bs, False
    else:
        lens, is_decode = [int(v) for v in rng.integers(0, 9, bs)], False
    s = sum(lens)
    V = 1000
    ids = torch.tensor(rng.integers(-3, V + 4, s), dtype=torch.int64)
    A_emb = torch.randn(L, R, V).to(torch.bfloat16)
    scal = [float(v) for v in rng.uniform(0.5, 2.0, L)]
    b = Batch(name, 0, lens, slots, is_decode, L, ranks, scal, 128)
    sgg = _sgg()
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    info, e = be.prepare_lora_batch_with_embedding(
        None if is_decode else lens, slots, ranks, scal, ids.to(DEV), A_emb.to(DEV), V,
        is_decode=is_decode)
    torch.cuda.synchronize()
    stg = be._staging
    assert list(stg.flag_view) == stg.seq   # the upload raised its done flag
    want = ol.embedding_a(ids.numpy(), to_f64(A_emb), lens, slots, ranks, V)
    assert np.array_equal(to_f64(e), want)
    check_plan(info, b, 128)
    assert info.lora_ranks.cpu().tolist() == list(ranks)
    assert info.req_weight_indices.cpu().tolist() == slots
    assert np.array_equal(info.scalings.cpu().numpy(), np.asarray(scal, np.float32))
    ref = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    rinfo = plan_on(ref, b)
    torch.cuda.synchronize()
    for f in ("permutation", "seg_indptr", "weight_indices", "req_seg_indptr",
              "req_weight_indices", "lora_ranks", "scalings", "work_indptr", "work_slots"):
        assert torch.equal(getattr(info, f), getattr(rinfo, f)), f
    assert (info.num_segments, info.max_len, info.num_work_segments) == \
        (rinfo.num_segments, rinfo.max_len, rinfo.num_work_segments)
    with pytest.raises(ValueError, match="ids"):
        be.prepare_lora_batch_with_embedding(None if is_decode else lens, slots, ranks, scal,
                                             ids[:-1].to(DEV), A_emb.to(DEV), V,
                                             is_decode=is_decode)


@pytest.mark.parametrize("seed", range(12))
def test_plan_upload_embedding_random(seed):
    """Seeded random batches through prepare_lora_batch_with_embedding:
    decode mode, one-token extend batches and mixed lengths; 1-80 slots
    (the one-launch form takes at most 64), ranks anywhere in [0, R + 8],
    R of 8-64, ids partly out of vocabulary.  Embedding rows bit-exact
    against the oracle, every plan region equal to the plain upload's."""
    sgg = _sgg()
    rng = np.random.default_rng(9000 + seed)
    L = int(rng.integers(1, 81))
    R = int(rng.choice([8, 16, 32, 64]))
    bs = int(rng.integers(1, 700))
    kind = ["decode", "ones", "mixed"][seed % 3]
    lens = [1] * bs if kind != "mixed" else [int(v) for v in rng.integers(0, 5, bs)]
    is_decode = kind == "decode"
    slots = [int(v) for v in rng.integers(0, L, bs)]
    ranks = [int(v) for v in rng.integers(0, R + 9, L)]
    scal = [float(v) for v in rng.uniform(0.25, 2.0, L)]
    V = 500
    s = sum(lens)
    ids = torch.tensor(rng.integers(-4, V + 5, s), dtype=torch.int64)
    A_emb = torch.randn(L, R, V).to(torch.bfloat16)
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    info, e = be.prepare_lora_batch_with_embedding(
        None if is_decode else lens, slots, ranks, scal, ids.to(DEV), A_emb.to(DEV), V,
        is_decode=is_decode)
    ref = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    rinfo = ref.prepare_lora_batch(None if is_decode else lens, slots, ranks, scal,
                                   is_decode=is_decode)
    torch.cuda.synchronize()
    want = ol.embedding_a(ids.numpy(), to_f64(A_emb), lens, slots, ranks, V)
    assert np.array_equal(to_f64(e), want)
    for f in ("permutation", "seg_indptr", "weight_indices", "req_seg_indptr",
              "req_weight_indices", "lora_ranks", "scalings", "work_indptr", "work_slots"):
        assert torch.equal(getattr(info, f), getattr(rinfo, f)), f


def test_plan_upload_embedding_graph_capacity():
    """The one-call upload + embedding into the graph-capacity plan buffer
    (init_cuda_graph_batch_info, a batch below the capacity): the embedding
    rows are the oracle's and every plan region is what
    prepare_lora_batch(use_cuda_graph=True) writes."""
    sgg = _sgg()
    rng = np.random.default_rng(77)
    L, V, R, bs, cap_bs = 8, 1000, 16, 200, 256
    slots = rng.integers(0, L, bs).tolist()
    ranks = [16, 8, 0, 16, 4, 16, 1, 16]
    scal = rng.uniform(0.5, 2.0, L).astype(np.float32).tolist()
    ids = torch.tensor(rng.integers(-3, V + 4, bs), dtype=torch.int64)
    A_emb = torch.randn(L, R, V).to(torch.bfloat16)
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    ref = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    be.init_cuda_graph_batch_info(cap_bs, 1)
    ref.init_cuda_graph_batch_info(cap_bs, 1)
    _, e = be.prepare_lora_batch_with_embedding(None, slots, ranks, scal, ids.to(DEV),
                                                A_emb.to(DEV), V, is_decode=True,
                                                use_cuda_graph=True)
    ref.prepare_lora_batch(None, slots, ranks, scal, is_decode=True, use_cuda_graph=True)
    torch.cuda.synchronize()
    want = ol.embedding_a(ids.numpy(), to_f64(A_emb), [1] * bs, slots, ranks, V)
    assert np.array_equal(to_f64(e), want)
    cap = be._graph_cap[2]
    assert _plan_regions(be, bs, bs, cap) == _plan_regions(ref, bs, bs, cap)


@pytest.mark.parametrize("form", ["separate", "one_call"])
def test_staging_ring_reuse_while_gpu_lags(form):
    """More batches than staging slots are planned while a delay kernel holds
    the stream, so the host must wait for each slot's done flag before
    reusing it; every batch's embedding gather (enqueued right after its
    upload, or in the same launch for the decode-shaped batches of the
    one-call form) must still see its own plan."""
    rng = np.random.default_rng(44)
    L, V, Re = 4, 300, 16
    ranks = [16, 8, 0, 16]
    A_emb = torch.randn(L, Re, V).to(torch.bfloat16)
    A_dev = A_emb.to(DEV)
    be = _sgg().ChunkedSgmvLoRA(L, 128, DEV)
    cases = []
    for i in range(30):
        bs = int(rng.integers(1, 13))
        lens = [int(v) for v in rng.integers(1, 41, bs)]
        if form == "one_call" and i % 2 == 0:
            lens = [1] * int(rng.integers(1, 300))   # decode-shaped: one launch
            bs = len(lens)
        slots = [int(v) for v in rng.integers(0, L, bs)]
        ids = torch.as_tensor(rng.integers(-5, V + 5, sum(lens)), dtype=torch.int64)
        cases.append([lens, slots, ids, ids.to(DEV)])
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)   # tens of milliseconds: the host runs ahead
    for i, case in enumerate(cases):
        if form == "separate":
            be.prepare_lora_batch(case[0], case[1], ranks, [1.0] * L)
            case[3] = be.run_lora_a_embedding(case[3], A_dev, V)
        else:
            case[3] = be.prepare_lora_batch_with_embedding(case[0], case[1], ranks, [1.0] * L,
                                                           case[3], A_dev, V)[1]
    torch.cuda.synchronize()
    stg = be._staging
    assert list(stg.flag_view) == stg.seq   # every upload raised its flag
    for lens, slots, ids, e in cases:
        want = ol.embedding_a(ids.numpy(), to_f64(A_emb), lens, slots, ranks, V)
        assert np.array_equal(to_f64(e), want)


def test_staging_wait_gives_up_on_a_flag_never_raised():
    """Host logic only: a slot whose upload never ran raises instead of spinning."""
    stg = _sgg().ChunkedSgmvLoRA(2, 128, DEV)._staging
    with pytest.raises(RuntimeError, match="has not run"):
        stg._wait(0, 7, limit_s=0.05)


def test_binding_rejects_outputs_too_small():
    """Host-side checks: an output (or h) with too few rows or columns is
    refused before anything is launched."""
    sgg = _sgg()
    b, proj, t = _small_case(41, [10, 6], [0, 1], 2, [8, 8], [2.0, 1.0], 256, [0, 256], 8)
    be = backend(b)
    info = plan_on(be, b)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    h = torch.zeros((16, 8), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="out has shape"):
        sgg.lora_shrink(x, A, info, 1, out=torch.zeros((15, 8), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="out has shape"):
        sgg.lora_shrink(x, A, info, 1, out=torch.zeros((16, 4), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="base_output has shape"):
        sgg.lora_expand(h, Bw, info, [0, 256], 256, base[:, :200])
    with pytest.raises(ValueError, match="h has shape"):
        sgg.lora_expand(h[:, :4], Bw, info, [0, 256], 256, base.clone())
    ids = torch.zeros(16, dtype=torch.int64, device=DEV)
    A_emb = torch.zeros((2, 8, 100), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="out has shape"):
        sgg.lora_a_embedding(ids, A_emb, info, 100,
                             out=torch.zeros((8, 8), dtype=torch.bfloat16, device=DEV))


def test_missing_base_gives_delta():
    b, proj, t = _small_case(40, [10, 6], [0, 1], 2, [8, 8], [2.0, 1.0], 256, [0, 256], 8)
    be = backend(b)
    plan_on(be, b)
    x, A, Bw = (t[k].to(DEV) for k in ("x", "A", "B"))
    y = be.run_lora_b_sgemm(be.run_lora_a_sgemm(x, A), Bw, [0, 256], None)
    t0 = dict(t, base=torch.zeros_like(t["base"]))
    _, want = oracle_forward(t0, b, proj)
    assert_close(y, want, "delta only")


def test_graph_mode_replays_match_oracle():
    """Capacity plan + captured kernels, replayed with different batches.

    The plan upload runs eagerly before each replay (as on the pages' graph
    path); base is reset eagerly, and every replay is checked on its own.
    """
    sgg = _sgg()
    L, K, R, offs, Re, V = 6, 512, 16, [0, 256, 320, 384], 16, 1000
    max_bs = 64
    rng = np.random.default_rng(55)
    proto = Batch("graph", 5555, [1] * max_bs, [0] * max_bs, True, L, [16, 16, 8, 0, 16, 16],
                  [1.0, 0.5, 2.0, 1.0, 1.5, 1.0], 128, [Projection("qkv", K, offs, R)])
    proj = proto.projections[0]
    t = draw_projection(proto, proj)
    x, A, Bw = (t[k].to(DEV) for k in ("x", "A", "B"))
    base0 = t["base"].to(DEV)
    base = base0.clone()
    A_emb = torch.randn(L, Re, V).to(torch.bfloat16)
    ids = torch.as_tensor(rng.integers(0, V, size=max_bs), dtype=torch.int64)
    ids_d, A_emb_d = ids.to(DEV), A_emb.to(DEV)
    h = torch.empty(max_bs, 3 * R, dtype=torch.bfloat16, device=DEV)
    e = torch.empty(max_bs, Re, dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device=DEV)
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    info = be.init_cuda_graph_batch_info(max_bs, 1)

    def kernels():
        sgg.lora_shrink(x, A, info, 3, out=h, workspace=ws)
        sgg.lora_expand(h, Bw, info, offs, 256, base)
        sgg.lora_a_embedding(ids_d, A_emb_d, info, V, out=e)

    be.prepare_lora_batch(None, [0] * max_bs, proto.lora_ranks, proto.scalings, is_decode=True,
                          use_cuda_graph=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kernels()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kernels()
    torch.cuda.synchronize()
    for trial in range(4):
        slots = rng.integers(0, L, size=max_bs).tolist()
        be.prepare_lora_batch(None, slots, proto.lora_ranks, proto.scalings, is_decode=True,
                              use_cuda_graph=True)
        base.copy_(base0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        b = Batch("g", 0, [1] * max_bs, slots, True, L, proto.lora_ranks, proto.scalings, 128,
                  proto.projections)
        want_h, want_y = oracle_forward(t, b, proj)
        assert_close(h, want_h, f"graph replay {trial} h")
        assert_close(base, want_y, f"graph replay {trial} y")
        want_e = ol.embedding_a(ids.numpy(), to_f64(A_emb), b.seq_lens, slots, b.lora_ranks, V)
        assert np.array_equal(to_f64(e), want_e), f"graph replay {trial} embedding"
        # eager work between replays, on the default stream
        torch.mm(torch.randn(64, 64, device=DEV), torch.randn(64, 64, device=DEV))


# ----------------------------------------------------------- device planner

def _plan_regions(be, s, bs, cap):
    """The meaningful contents of the graph plan buffer, region by region."""
    v = be.cuda_graph_batch_info
    return {"permutation": v.permutation[:s].cpu().tolist(),
            "seg_indptr": v.seg_indptr[:cap + 1].cpu().tolist(),
            "seg_slots": v.weight_indices[:cap].cpu().tolist(),
            "req_seg_indptr": v.req_seg_indptr[:bs + 1].cpu().tolist(),
            "req_slots": v.req_weight_indices[:bs].cpu().tolist(),
            "ranks": v.lora_ranks.cpu().tolist(),
            "scalings": v.scalings.cpu().tolist(),
            "work_indptr": v.work_indptr[:cap + 1].cpu().tolist(),
            "work_slots": v.work_slots[:cap].cpu().tolist()}


DEVICE_PLAN_CASES = [
    # (name, bs, max_bs, tokens_per_bs, L, lens (None: decode), max_chunk, override)
    ("decode256", 256, 256, 1, 8, None, 128, 0),
    ("decode3000_L700", 3000, 3000, 1, 700, None, 128, 0),
    ("extend_zero_lens", 100, 128, 300, 37, (0, 300), 128, 0),
    ("override3", 50, 64, 200, 5, (0, 20), 128, 3),
    ("override48", 60, 64, 200, 4, (0, 200), 128, 48),
    ("cap16", 40, 40, 100, 6, (1, 100), 16, 0),
    ("L1024_bs4096", 4096, 4096, 3, 1024, (0, 3), 128, 0),
    ("decode_L1024_bs4096", 4096, 4096, 1, 1024, None, 128, 0),
    ("unit_L1024_bs4096", 4096, 4096, 1, 1024, (1, 1), 128, 0),
    # slot counts around the one- and two-wave slot scans (64, 128)
    ("decode500_L64", 500, 512, 1, 64, None, 128, 0),
    ("decode500_L65", 500, 512, 1, 65, None, 128, 0),
    ("extend_L100", 120, 128, 40, 100, (0, 40), 128, 0),
    ("decode700_L128", 700, 700, 1, 128, None, 128, 0),
    ("extend_L129", 150, 160, 30, 129, (1, 30), 32, 0),
]


def _random_device_plan_cases(n=10):
    """Seeded random batches for the device planner: one-token requests
    (decode mode, or extend mode with every length 1 -- the placement's
    bit-matching path) and extend batches, slot counts 1..1024."""
    rng = np.random.default_rng(4242)
    out = []
    for i in range(n):
        L = int(rng.choice([1, 2, 3, 64, 65, 511, 512, 1023, 1024, int(rng.integers(1, 1025))]))
        bs = int(rng.integers(1, 4097))
        kind = i % 3
        lens = None if kind == 0 else ((1, 1) if kind == 1 else (0, 5))
        tpb = 1 if lens is None else lens[1]
        cap = int(rng.choice([16, 32, 64, 128]))
        override = int(rng.choice([0, 0, 16, 48]))   # the graph capacity assumes chunks >= 16
        out.append((f"random{i}_L{L}_bs{bs}", bs, bs, tpb, L, lens, cap, override))
    return out


DEVICE_PLAN_CASES += _random_device_plan_cases()


@pytest.mark.parametrize("case", DEVICE_PLAN_CASES, ids=[c[0] for c in DEVICE_PLAN_CASES])
def test_device_plan_matches_host_plan(case):
    """lora_plan_device writes, bit for bit, the plan the host planner uploads
    for the same batch and capacities, and that plan is the oracle's."""
    sgg = _sgg()
    name, bs, max_bs, tpb, L, lens_rng, max_chunk, override = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    decode = lens_rng is None
    lens = [1] * bs if decode else rng.integers(lens_rng[0], lens_rng[1] + 1, bs).tolist()
    slots = rng.integers(0, L, bs).tolist()
    ranks = rng.integers(0, 65, L).tolist()
    scal = rng.uniform(0, 4, L).astype(np.float32).tolist()
    hb = sgg.ChunkedSgmvLoRA(L, max_chunk, DEV)
    db = sgg.ChunkedSgmvLoRA(L, max_chunk, DEV)
    hb.init_cuda_graph_batch_info(max_bs, tpb)
    db.init_cuda_graph_batch_info(max_bs, tpb)
    _, max_tokens, cap = hb._graph_cap
    hb.prepare_lora_batch(None if decode else lens, slots, ranks, scal, is_decode=decode,
                          use_cuda_graph=True, chunk_size_override=override)
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=DEV)
    db.prepare_lora_batch_device(None if decode else i32(lens), i32(slots), i32(ranks),
                                 torch.tensor(scal, dtype=torch.float32, device=DEV),
                                 is_decode=decode, chunk_size_override=override)
    torch.cuda.synchronize()
    s = sum(lens)
    got, want = _plan_regions(db, s, bs, cap), _plan_regions(hb, s, bs, cap)
    for k in want:
        assert got[k] == want[k], k
    ref = op.plan(None if decode else lens, slots, decode, max_chunk, override, capacity=cap)
    assert got["permutation"] == ref["permutation"]
    assert got["seg_indptr"] == ref["seg_indptr"] and got["seg_slots"] == ref["seg_slots"]
    info = db.cuda_graph_plan_info.cpu().tolist()
    assert info[6] == 0
    assert info[0] == ref["num_segments"] and info[1] == ref["chunk_size"] and info[3] == s


@pytest.mark.parametrize("bad", ["slot", "negative_len", "decode_bad_slot", "too_many_tokens"])
def test_device_plan_invalid_batch_is_empty(bad):
    """An invalid batch found on the device is not planned: a non-zero status
    and every segment empty, so the kernels that follow do nothing."""
    sgg = _sgg()
    L, bs = 4, 16
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    be.init_cuda_graph_batch_info(bs, 8)
    _, max_tokens, cap = be._graph_cap
    lens, slots, decode = [3] * bs, [1] * bs, False
    if bad == "slot":
        slots[5] = L
    elif bad == "negative_len":
        lens[2] = -1
    elif bad == "decode_bad_slot":
        decode, lens = True, [1] * bs
        slots[0] = -1
    elif bad == "too_many_tokens":
        lens[0] = max_tokens
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=DEV)
    lens_d = i32(lens)
    be.prepare_lora_batch_device(None if decode else lens_d, i32(slots), i32([8] * L),
                                 torch.ones(L, dtype=torch.float32, device=DEV), is_decode=decode)
    torch.cuda.synchronize()
    v = be.cuda_graph_batch_info
    assert be.cuda_graph_plan_info[6].item() != 0
    assert v.seg_indptr[:cap + 1].cpu().tolist() == [0] * (cap + 1)
    assert v.work_indptr[:cap + 1].cpu().tolist() == [0] * (cap + 1)


@pytest.mark.parametrize("form", ["separate", "stacked"])
def test_device_plan_captured_with_kernels(form):
    """The device planner captured in one graph with the shrink and the
    expand (separate calls, or the stacked call as the decode step runs it);
    the lengths and slots are rewritten in device memory before each replay,
    and every replay is checked against the oracle."""
    sgg = _sgg()
    L, K, R, offs = 5, 512, 16, [0, 256, 320, 384]
    max_bs, tpb = 24, 12
    rng = np.random.default_rng(77)
    ranks, scal = [16, 8, 0, 16, 12], [1.0, 0.5, 2.0, 1.5, 1.0]
    proto = Batch("devgraph", 7777, [tpb] * max_bs, [0] * max_bs, False, L, ranks, scal, 128,
                  [Projection("qkv", K, offs, R)])
    proj = proto.projections[0]
    t = draw_projection(proto, proj)
    x, A, Bw = (t[k].to(DEV) for k in ("x", "A", "B"))
    base0 = t["base"].to(DEV)
    base = base0.clone()
    h = torch.empty(max_bs * tpb, 3 * R, dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device=DEV)
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    info = be.init_cuda_graph_batch_info(max_bs, tpb)
    lens_d = torch.full((max_bs,), tpb, dtype=torch.int32, device=DEV)
    slots_d = torch.zeros(max_bs, dtype=torch.int32, device=DEV)
    ranks_d = torch.tensor(ranks, dtype=torch.int32, device=DEV)
    scal_d = torch.tensor(scal, dtype=torch.float32, device=DEV)

    def step():
        be.prepare_lora_batch_device(lens_d, slots_d, ranks_d, scal_d)
        if form == "stacked":
            sgg.lora_qkv(x, A, Bw, info, offs, 256, base, workspace=ws)
        else:
            sgg.lora_shrink(x, A, info, 3, out=h, workspace=ws)
            sgg.lora_expand(h, Bw, info, offs, 256, base)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for trial in range(4):
        lens = rng.integers(0, tpb + 1, max_bs).tolist()
        slots = rng.integers(0, L, max_bs).tolist()
        lens_d.copy_(torch.tensor(lens, dtype=torch.int32))
        slots_d.copy_(torch.tensor(slots, dtype=torch.int32))
        base.copy_(base0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert be.cuda_graph_plan_info[6].item() == 0
        s = sum(lens)
        b = Batch("g", 0, lens, slots, False, L, ranks, scal, 128, proto.projections)
        ts = {"x": t["x"][:s], "A": t["A"], "B": t["B"], "base": t["base"][:s]}
        want_h, want_y = oracle_forward(ts, b, proj)
        if form == "separate":
            assert_close(h[:s], want_h, f"device-planned replay {trial} h")
        assert_close(base[:s], want_y, f"device-planned replay {trial} y ({form})")
        # rows past the batch's tokens are not touched
        assert torch.equal(base[s:].view(torch.int16), base0[s:].view(torch.int16))


@pytest.mark.parametrize("lens", [[3, 0, 5, 2, 7], [400, 0, 500, 600, 700]],
                         ids=["small", "large"])
def test_plan_upload_from_pageable_staging(lens):
    """lora_plan_upload with a staging buffer that has no device mapping
    (pageable memory) takes the runtime-copy path and still raises the done
    flag; every region of the uploaded plan is the oracle's or the input's."""
    from segmented_gather_gemm_amd import _lib
    slots, L = [2, 1, 0, 2, 1], 3
    ranks = np.array([8, 16, 4], np.int32)
    scal = np.array([1.0, 0.5, 2.0], np.float32)
    s, bs = sum(lens), len(lens)
    cap = int(_lib.lib().lora_plan_max_segments(s, L, 16))
    offs = (ctypes.c_int64 * 10)()
    total = int(_lib.lib().lora_plan_layout(s, cap, bs, L, offs))
    staging = np.zeros(total, np.int32)            # pageable host memory
    dev = torch.zeros(total, dtype=torch.int32, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    info = np.zeros(6, np.int32)
    rc = _lib.calls().lora_plan_upload(
        np.array(lens, np.int32), np.array(slots, np.int32), bs, ranks, scal, L, 0, 128, 0, s,
        cap, bs, staging, dev.data_ptr(), 4 * total, info, flag.data_ptr(), 7,
        torch._C._cuda_getCurrentRawStream(0))
    assert rc == 0, _lib.lib().lora_last_error()
    torch.cuda.synchronize()
    assert flag.item() == 7
    ref = op.plan(lens, slots, False, 128, capacity=cap)
    got = dev.cpu().numpy()
    assert got[offs[0]:offs[0] + s].tolist() == ref["permutation"]
    assert got[offs[1]:offs[1] + cap + 1].tolist() == ref["seg_indptr"]
    assert got[offs[2]:offs[2] + cap].tolist() == ref["seg_slots"]
    assert got[offs[3]:offs[3] + bs + 1].tolist() == ref["req_seg_indptr"]
    assert got[offs[4]:offs[4] + bs].tolist() == slots
    assert got[offs[5]:offs[5] + L].tolist() == ranks.tolist()
    assert got[offs[6]:offs[6] + L].view(np.float32).tolist() == scal.tolist()
    assert info[0] == ref["num_segments"] and info[1] == ref["chunk_size"] and info[3] == s


# ------------------------------------------------------------- MoE LoRA add

def _moe_case(seed, lens, L, ranks, E, k, K, N, R, bad_experts=0):
    """A batch planned by the backend plus MoE routing and weights (bf16):
    topk_ids (s, k) with `bad_experts` entries out of range."""
    rng = np.random.default_rng(seed)
    bs = len(lens)
    slots = rng.integers(0, L, size=bs).tolist()
    scal = rng.uniform(0.5, 2.0, size=L).tolist()
    s = int(sum(lens))
    topk = rng.integers(0, E, size=(s, k)).astype(np.int32)
    for i in range(bad_experts):
        topk[rng.integers(0, s), rng.integers(0, k)] = [-1, E, E + 7][i % 3]
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)
    t = {"x": bf(rng.standard_normal((s, K))),
         "A": bf(rng.standard_normal((L, E, R, K)) * 0.02),   # N(0, 0.02^2), as the workloads
         "B": bf(rng.standard_normal((L, E, N, R)) * 0.02),
         "out": bf(rng.standard_normal((s * k, N)))}
    return slots, scal, topk, t


def _moe_want(t, lens, slots, ranks, scal, topk, E):
    """Oracle result; rows of out-of-range experts keep their values."""
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ok = (topk >= 0) & (topk < E)
    want = om.moe_lora_add(to_f64(t["x"]), to_f64(t["A"]), to_f64(t["B"]), to_f64(t["out"]),
                           indptr, slots, np.where(ok, topk, 0), ranks, scal)
    keep = ~ok.reshape(-1)
    want[keep] = to_f64(t["out"])[keep]
    return want, indptr


@pytest.mark.parametrize("case", [
    ("extend", [3, 1, 5, 2, 1, 4, 37, 60, 9, 128], 4, [16, 8, 0, 16], 8, 2, 512, 256, 16, 0),
    ("decode", [1] * 300, 6, [16, 16, 12, 8, 16, 4], 8, 2, 1024, 384, 16, 0),
    ("top4_bad_experts", [2, 7, 1, 30, 5], 3, [32, 0, 24], 4, 4, 256, 136, 32, 5),
    # the shape bench.py times: 256 decode tokens, top-2 of 8 experts, 4096 -> 14336
    ("bench_shape", [1] * 256, 8, [16] * 8, 8, 2, 4096, 14336, 16, 0),
], ids=lambda c: c[0])
def test_moe_lora_add_matches_oracle(case):
    """Per-request routing to virtual experts (bit-exact against the oracle)
    and the copies planned on the GPU in one launch (lora_moe_plan), and the
    MoE LoRA add
    into the fused-MoE intermediate against the oracle; copies whose expert
    id is out of range keep their rows bit for bit."""
    name, lens, L, ranks, E, k, K, N, R, bad = case
    sgg = _sgg()
    slots, scal, topk, t = _moe_case(zlib.crc32(name.encode()) % 1000, lens, L, ranks, E, k, K,
                                     N, R, bad_experts=bad)
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    decode = name in ("decode", "bench_shape")
    be.prepare_lora_batch(None if decode else lens, slots, ranks, scal, is_decode=decode)
    topk_d = torch.from_numpy(topk).to(DEV)
    info = be.prepare_moe_lora_batch(topk_d, E)
    out = t["out"].to(DEV)
    be.run_moe_lora_add(t["x"].to(DEV), t["A"].to(DEV), t["B"].to(DEV), out, k)
    torch.cuda.synchronize()
    assert int(be.moe_plan_info[6].item()) == 0, "the copies' plan was rejected"
    want, indptr = _moe_want(t, lens, slots, ranks, scal, topk, E)
    ok = (topk >= 0) & (topk < E)
    v_want = om.virtual_experts(indptr, slots, np.where(ok, topk, 0), E)
    v_want[~ok.reshape(-1)] = L * E
    got_v = info.req_weight_indices[:len(topk) * k].cpu().numpy()
    assert np.array_equal(got_v, v_want)
    assert info.lora_ranks.cpu().tolist() == [r for r in ranks for _ in range(E)] + [0]
    assert np.array_equal(info.scalings.cpu().numpy(),
                          np.append(np.repeat(np.asarray(scal, np.float32), E), 0))
    keep = ~ok.reshape(-1)
    assert torch.equal(out[torch.from_numpy(keep).to(DEV)].view(torch.int16),
                       t["out"][torch.from_numpy(keep)].to(DEV).view(torch.int16))
    assert_close(out, want, f"MoE LoRA add ({name})")


@pytest.mark.parametrize("case", [
    ("extend", [3, 1, 5, 2, 1, 4, 37, 60, 9, 128], 4, [16, 8, 0, 16], 8, 2, 0, 0),
    ("decode_bad_experts", [1] * 300, 6, [16, 16, 12, 8, 16, 4], 8, 2, 7, 0),
    ("top4", [2, 7, 1, 30, 5], 3, [32, 0, 24], 4, 4, 5, 0),
    ("limits_4096_copies_1017_slots", [1] * 2048, 8, [16] * 8, 127, 2, 3, 0),
    ("tokens_past_the_requests", [4, 6, 2], 3, [16, 8, 4], 5, 2, 0, 9),
], ids=lambda c: c[0])
def test_moe_plan_one_launch_matches_route_then_plan(case):
    """lora_moe_plan gives every region of the copies' plan, the virtual
    tables and the info words bit for bit as lora_moe_route followed by
    lora_plan_device; copies of tokens outside every request (the request
    boundaries end early) go to the extra virtual slot in both."""
    from segmented_gather_gemm_amd import binding as Bn
    name, lens, L, ranks, E, k, bad, extra_tokens = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    slots = rng.integers(0, L, size=len(lens)).astype(np.int32)
    scal = rng.uniform(0.5, 2.0, size=L).astype(np.float32)
    s = int(sum(lens)) + extra_tokens
    topk = rng.integers(0, E, size=(s, k)).astype(np.int32)
    for i in range(bad):
        topk[rng.integers(0, s), rng.integers(0, k)] = [-1, E, E + 7][i % 3]
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    indptr_d, slots_d, topk_d = d(indptr), d(slots), d(topk)
    ranks_d, scal_d = d(np.asarray(ranks, np.int32)), d(scal)
    copies, nv = s * k, L * E + 1
    lib = _sgg()._lib.lib()
    seg_cap = int(lib.lora_plan_max_segments(copies, nv, 16))
    offs = (ctypes.c_int64 * 10)()
    total = int(lib.lora_plan_layout(copies, seg_cap, copies, nv, offs))
    plans = [torch.full((total,), -7, dtype=torch.int32, device=DEV) for _ in range(2)]
    infos = [torch.full((8,), -7, dtype=torch.int32, device=DEV) for _ in range(2)]
    vslots = torch.empty(copies, dtype=torch.int32, device=DEV)
    vranks = torch.empty(nv, dtype=torch.int32, device=DEV)
    vscal = torch.empty(nv, dtype=torch.float32, device=DEV)
    Bn.lora_moe_route(indptr_d, slots_d, len(lens), topk_d, E, ranks_d, scal_d, L, vslots,
                      vranks, vscal)
    Bn.lora_plan_device(None, vslots, vranks, vscal, nv, True, 128, 0, copies, seg_cap, copies,
                        plans[0], infos[0])
    Bn.lora_moe_plan(indptr_d, slots_d, len(lens), topk_d, E, ranks_d, scal_d, L, 128, seg_cap,
                     plans[1], infos[1])
    torch.cuda.synchronize()
    assert torch.equal(infos[0], infos[1]) and int(infos[1][6]) == 0
    assert torch.equal(plans[0][:offs[9]], plans[1][:offs[9]])
    got = plans[1].cpu().numpy()
    assert got[offs[5]:offs[5] + nv].tolist() == vranks.cpu().tolist()
    assert np.array_equal(got[offs[6]:offs[6] + nv].view(np.float32), vscal.cpu().numpy())
    ok = (topk >= 0) & (topk < E)
    inside = int(sum(lens))   # tokens past the last request have none: the extra slot
    v_want = np.full(copies, L * E, dtype=np.int64)
    v_want[:inside * k] = om.virtual_experts(indptr.astype(np.int64), slots.tolist(),
                                             np.where(ok, topk, 0)[:inside], E)
    v_want[~ok.reshape(-1)] = L * E
    assert np.array_equal(got[offs[4]:offs[4] + copies], v_want)


def test_moe_lora_add_in_a_graph():
    """Routing, the GPU plan of the copies and the add captured in one graph;
    replays with new router choices written into the captured topk tensor,
    eager work between them, each checked against the oracle."""
    sgg = _sgg()
    lens, L, ranks, E, k, K, N, R = [1] * 200, 4, [16, 8, 16, 0], 8, 2, 512, 256, 16
    slots, scal, topk, t = _moe_case(5, lens, L, ranks, E, k, K, N, R)
    be = sgg.ChunkedSgmvLoRA(L, 128, DEV)
    be.prepare_lora_batch(None, slots, ranks, scal, is_decode=True)
    topk_d = torch.from_numpy(topk).to(DEV)
    x, A, Bw = t["x"].to(DEV), t["A"].to(DEV), t["B"].to(DEV)
    out0 = t["out"].to(DEV)
    out = out0.clone()
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device=DEV)

    def step():
        info = be.prepare_moe_lora_batch(topk_d, E)
        sgg.lora_moe_add(x, A, Bw, info, k, out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    for trial in range(3):
        topk = rng.integers(0, E, size=topk.shape).astype(np.int32)
        topk_d.copy_(torch.from_numpy(topk))
        out.copy_(out0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want, _ = _moe_want(t, lens, slots, ranks, scal, topk, E)
        assert_close(out, want, f"MoE graph replay {trial}")
        torch.mm(torch.randn(64, 64, device=DEV), torch.randn(64, 64, device=DEV))
