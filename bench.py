"""Benchmark: chunked SGMV LoRA hot path on one MI355X.

A step is one pass of the whole path over one batch: host plan (native
planner) -> one async upload of the plan -> LoRA-A shrink -> LoRA-B expand
(scaling, stacked slice offsets, in place into base) -> LoRA-A embedding
gather.  The timed steps are eager: one native call plans, uploads and runs
the embedding gather (one launch for a decode batch), one runs lora_qkv (the
stacked shrink and expand).  The same step with the upload and the gather as
separate calls, and graph mode, are timed too and reported beside it.  The headline
workload is the decode batch: 256 one-token requests on 8 adapters drawn
uniformly, rank 16, stacked qkv 4096 -> [4096, 1024, 1024], bf16; the
embedding gather uses vocab 128256 and rank 16.  Inputs rotate over 48
independent sets (> the 256 MB MALL) so kernels read HBM, not cache.

Prints ONE JSON line.  `value` is tokens/s of whole steps (wall clock over
the timed steps, inputs resident in HBM); kernel durations come from HIP
events on the stream the kernels run on.  Every run also times the other
workloads, each under its own key: the prefill chunk sweep (16 / 32 / 64 /
128), the skewed batch (o_proj, down_proj), the Llama-3-8B-shaped layer
sweep with the embedding gather, the pruned lm_head pass of the decode batch,
the device-side planner, the shrink's MFMA and VALU forms on short segments,
the MoE LoRA add and decode-shaped batches of 1024-16384 tokens; `--legs`
picks some, `--quick` skips them all.
"""

import argparse
import ctypes
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_prefill_kernels_hbm_traffic.txt")
LEGS = ("prefill", "skewed", "full", "lm_head", "device_plan", "short", "moe", "decode_sizes")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=48, help="rotated input sets")
    ap.add_argument("--quick", action="store_true",
                    help="time the decode step only (skip the prefill chunk sweep, the skewed "
                         "batch, the full layer sweep, the lm_head pass and the device planner)")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma list of the workloads timed after the decode step "
                         "(prefill, skewed, full, lm_head, device_plan; empty for none)")
    ap.add_argument("--full-layers", type=int, default=4,
                    help="resident layers with distinct weights in the full layer sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--fused-timeline", action="store_true",
                    help="only record the one-launch stacked call's per-workgroup timeline on "
                         "the decode batch (the library's fused_trace option) and print it")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (for counter calibration)")
    return ap.parse_args()


# ----------------------------------------------------------- algorithmic work

def algo_counts(b, proj, emb_rank):
    """Algorithmic bytes / flops of each kernel for one batch (padding and
    zero-fill not counted): x read once, each active adapter's weights read
    once, h written and read once, base read and written once."""
    ranks = np.asarray(b.lora_ranks)
    tok_rank = np.repeat(ranks[np.asarray(b.req_slots)], b.seq_lens).astype(np.int64)
    sum_rho = int(tok_rank.sum())
    active = sorted(set(b.req_slots))
    act_rho = int(sum(min(ranks[a], proj.rank) for a in active))
    s, K, c, N = b.num_tokens, proj.in_dim, proj.num_slices, proj.out_dim
    shrink_b = 2 * s * K + 2 * c * K * act_rho + 2 * c * sum_rho + 4 * s
    expand_b = 2 * c * sum_rho + 2 * N * act_rho + 4 * s * N + 4 * s
    emb_rho = np.minimum(tok_rank, emb_rank)
    emb_b = int(np.sum(8 + 4 + 4 * emb_rho))
    return {"shrink": {"bytes": shrink_b, "flops": 2 * K * c * sum_rho},
            "expand": {"bytes": expand_b, "flops": 2 * N * sum_rho},
            "embedding": {"bytes": emb_b, "flops": 0}}


def kernel_source_hash():
    """First 16 hex digits of sha256 over the sources of libsgg_lora.so (the
    planner, kernels and launch code; not the CPython call module)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "segmented_gather_gemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".cpp", ".h")):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed counter runs, if they were
    taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        rec[k.strip()] = v.strip()
    if rec.get("source_sha") != kernel_source_hash():
        return None
    key = f"{workload}.{kernel}.hbm_bytes_per_launch"
    return float(rec[key]) if key in rec else None


# ---------------------------------------------------------------- GPU legs

def make_sets(n_sets, device):
    import torch
    from synth import draw_batch, draw_embedding, draw_ids, draw_projection
    from synth.workloads import rotation_batch
    base_b = draw_batch("decode")
    # one LoRA-A embedding table (33 MB) shared by all sets; ids differ per set
    _, A_emb = draw_embedding(base_b)
    A_emb = A_emb.to(device)
    sets = []
    for i in range(n_sets):
        b = base_b if i == 0 else rotation_batch(base_b, i)
        proj = b.projections[0]
        t = draw_projection(b, proj)
        sets.append({"b": b, "proj": proj,
                     **{k: v.to(device) for k, v in t.items()},
                     "ids": draw_ids(b).to(device), "A_emb": A_emb,
                     "e": torch.empty((b.num_tokens, A_emb.shape[1]), dtype=torch.bfloat16,
                                      device=device)})
    return sets


def hold_stream(stream, ms):
    """Enqueue a delay kernel of about `ms` milliseconds on `stream`; return
    an event recorded after it (not yet complete while the delay runs)."""
    import torch
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            torch.cuda._sleep(1 << 22)
            b.record(stream)
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = (1 << 22) / max(a.elapsed_time(b), 1e-3)
    done = torch.cuda.Event()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))
        done.record(stream)
    return done


_SLEEP_CYCLES_PER_MS = None


def own_plan(info):
    """A copy of a batch plan whose device arrays belong to it alone."""
    import dataclasses
    import torch
    return dataclasses.replace(info, **{
        f.name: getattr(info, f.name).clone() for f in dataclasses.fields(info)
        if isinstance(getattr(info, f.name), torch.Tensor)})


def seg_histogram(info):
    """Plan segment lengths in power-of-two bins: {"1": n, "2-3": n, ..., "128+": n}."""
    n = info.num_segments
    lens = np.diff(info.seg_indptr[:n + 1].cpu().numpy().astype(np.int64))
    edges = [1, 2, 4, 8, 16, 32, 64, 128]
    out = {}
    for i, lo in enumerate(edges):
        hi = edges[i + 1] if i + 1 < len(edges) else None
        key = str(lo) if hi == lo + 1 else (f"{lo}-{hi - 1}" if hi else f"{lo}+")
        out[key] = int(((lens >= lo) & (lens < hi)).sum() if hi else (lens >= lo).sum())
    return out


def host_plan_us(be, b, max_chunk=None, n=50):
    """Host time of one plan + upload call (prepare_lora_batch), averaged."""
    import torch
    lens = None if b.is_decode else np.asarray(b.seq_lens, np.int32)
    slots = np.asarray(b.req_slots, np.int32)
    ranks, scal = np.asarray(b.lora_ranks, np.int32), np.asarray(b.scalings, np.float32)
    for _ in range(3):
        be.prepare_lora_batch(lens, slots, ranks, scal, is_decode=b.is_decode)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        be.prepare_lora_batch(lens, slots, ranks, scal, is_decode=b.is_decode)
    us = (time.perf_counter() - t0) / n * 1e6
    torch.cuda.synchronize()
    return round(us, 2)


def rotated(t, n):
    """n input sets for one projection: the drawn set, then copies whose
    values are rolled along K (x, A) or N (B, base) on the GPU, so every set
    is its own memory; rank padding rows and columns keep their places."""
    sets = [t]
    for i in range(1, n):
        sets.append({"x": t["x"].roll(8 * i, dims=1), "A": t["A"].roll(8 * i, dims=2),
                     "B": t["B"].roll(8 * i, dims=1), "base": t["base"].roll(8 * i, dims=1)})
    return sets


def run_decode(args, device):
    """Decode steps.  Headline (eager): the host plan, its upload and the
    embedding gather in one C call and one launch, then the stacked shrink +
    expand (lora_qkv).  Beside it: the same step with the upload and the
    gather as two calls, and graph mode (the gather and the stacked call's
    launches captured once per input set over a fixed-capacity plan,
    replayed after each plan upload)."""
    import torch
    import segmented_gather_gemm_amd as sgg

    sets = make_sets(args.sets, device)
    b0 = sets[0]["b"]
    vocab = b0.vocab_size or 128256
    stream = torch.cuda.current_stream(device)
    names = ("shrink", "expand", "embedding")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=device)
    for st in sets:
        st["h"] = torch.empty((st["b"].num_tokens, st["A"].shape[1]), dtype=torch.bfloat16,
                              device=device)
        st["slots"] = np.asarray(st["b"].req_slots, np.int32)
        st["ranks"] = np.asarray(st["b"].lora_ranks, np.int32)
        st["scal"] = np.asarray(st["b"].scalings, np.float32)

    # ---- eager steps (headline)
    be = sgg.ChunkedSgmvLoRA(b0.num_loras, b0.max_chunk_size, device)

    def eager_step(i):
        # plan + upload and the embedding gather in one C call (one launch)
        st = sets[i % len(sets)]
        proj = st["proj"]
        info = be.prepare_lora_batch_with_embedding(None, st["slots"], st["ranks"], st["scal"],
                                                    st["ids"], st["A_emb"], vocab,
                                                    is_decode=True, out=st["e"])[0]
        sgg.lora_qkv(st["x"], st["A"], st["B"], info, proj.slice_offsets, proj.max_slice,
                     st["base"], workspace=ws)

    def eager_step_separate(i):
        # the same step with the upload and the embedding gather as two calls
        st = sets[i % len(sets)]
        proj = st["proj"]
        info = be.prepare_lora_batch(None, st["slots"], st["ranks"], st["scal"], is_decode=True)
        sgg.lora_a_embedding(st["ids"], st["A_emb"], info, vocab, out=st["e"])
        sgg.lora_qkv(st["x"], st["A"], st["B"], info, proj.slice_offsets, proj.max_slice,
                     st["base"], workspace=ws)

    # Set-up leaves many young objects; a full collection of them inside the
    # timed steps would cost ~30 ms, so collect once before timing.
    gc.collect()
    # Priming, part of making the inputs resident: every input set goes
    # through the step once (first touch of its pages), repeated until the
    # GPU has been kept busy for ~50 ms, so a short timed run does not sit in
    # the clock ramp that follows the CPU-side set-up (measured: 20 steps
    # after 5 warm-up steps took 30-35 us per step cold, 26 us after 30 ms of
    # GPU work, 23 us in a 200-step run).
    t_prime = time.perf_counter()
    primed = 0
    while primed < len(sets) or time.perf_counter() - t_prime < 0.05:
        eager_step(primed)
        primed += 1
        if primed % len(sets) == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    prime_ms = (time.perf_counter() - t_prime) * 1e3
    for i in range(args.warmup):
        eager_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        eager_step(i)
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    for i in range(args.warmup):
        eager_step_separate(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        eager_step_separate(i)
    torch.cuda.synchronize()
    separate_wall = time.perf_counter() - t0

    # ---- kernel durations, same plans and launch configuration, HIP events
    # on the launch stream.  The plans are made first; then, per kernel, a
    # delay kernel holds the stream while one launch per step is queued
    # between two events, so the launches run back to back and the average
    # launch duration is the interval over the number of launches.
    # Every timed launch gets its own copy of its plan: the backend's ring
    # holds 8 live plans, and launch i must read set i's plan, not the plan
    # of a later batch that reused its ring slot.
    infos = []
    for i in range(args.steps):
        st = sets[i % len(sets)]
        infos.append(own_plan(be.prepare_lora_batch(None, st["slots"], st["ranks"], st["scal"],
                                                    is_decode=True)))
    torch.cuda.synchronize()

    def one(n, i):
        st, info = sets[i % len(sets)], infos[i]
        proj = st["proj"]
        if n == "qkv":
            sgg.lora_qkv(st["x"], st["A"], st["B"], info, proj.slice_offsets, proj.max_slice,
                         st["base"], workspace=ws)
        elif n == "embedding":
            sgg.lora_a_embedding(st["ids"], st["A_emb"], info, vocab, out=st["e"])
        elif n == "shrink":
            sgg.lora_shrink(st["x"], st["A"], info, proj.num_slices, out=st["h"], workspace=ws)
        else:
            sgg.lora_expand(st["h"], st["B"], info, proj.slice_offsets, proj.max_slice,
                            st["base"])

    dur = {}
    back_to_back = True
    for n in names + ("qkv", "qkv_one_launch"):
        fused = sgg.lora_set_option("fused_stacked", 1 if n == "qkv_one_launch" else 0)
        for i in range(min(args.warmup, args.steps)):
            one("qkv" if n == "qkv_one_launch" else n, i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        held = hold_stream(stream, 5.0 + 0.05 * args.steps)
        e0.record(stream)
        for i in range(args.steps):
            one("qkv" if n == "qkv_one_launch" else n, i)
        e1.record(stream)
        back_to_back &= not held.query()   # the delay outlasted the enqueueing
        torch.cuda.synchronize()
        sgg.lora_set_option("fused_stacked", fused)
        dur[n] = e0.elapsed_time(e1) * 1e3 / args.steps   # microseconds per launch
    del infos

    # the upload launch alone (plan copy) and with the embedding gather, one
    # per prepared batch, back to back: at most one ring's worth of batches,
    # so no prepare waits for a slot while the delay kernel holds the stream
    def prep(n, i):
        st = sets[i % len(sets)]
        if n == "copy":
            be.prepare_lora_batch(None, st["slots"], st["ranks"], st["scal"], is_decode=True)
        else:
            be.prepare_lora_batch_with_embedding(None, st["slots"], st["ranks"], st["scal"],
                                                 st["ids"], st["A_emb"], vocab, is_decode=True,
                                                 out=st["e"])
    n_up = min(args.steps, be._staging.n)
    # GPU time of whole eager steps: one ring's worth queued behind a delay
    # kernel (the host's planning hidden), against the wall-clock step
    for i in range(n_up):
        eager_step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    held = hold_stream(stream, 5.0)
    e0.record(stream)
    for i in range(n_up):
        eager_step(i)
    e1.record(stream)
    back_to_back &= not held.query()
    torch.cuda.synchronize()
    step_gpu_us = e0.elapsed_time(e1) * 1e3 / n_up
    upload = {"launches": n_up}
    for n in ("copy", "copy_and_embedding"):
        for i in range(n_up):
            prep(n, i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        held = hold_stream(stream, 5.0)
        e0.record(stream)
        for i in range(n_up):
            prep(n, i)
        e1.record(stream)
        back_to_back &= not held.query()
        torch.cuda.synchronize()
        upload[n + "_us"] = round(e0.elapsed_time(e1) * 1e3 / n_up, 3)

    # ---- graph mode (secondary)
    bg = sgg.ChunkedSgmvLoRA(b0.num_loras, b0.max_chunk_size, device)
    ginfo = bg.init_cuda_graph_batch_info(b0.num_tokens, 1)

    def launch_g(st):
        proj = st["proj"]
        sgg.lora_a_embedding(st["ids"], st["A_emb"], ginfo, vocab, out=st["e"])
        sgg.lora_shrink(st["x"], st["A"], ginfo, proj.num_slices, out=st["h"], workspace=ws)
        sgg.lora_expand(st["h"], st["B"], ginfo, proj.slice_offsets, proj.max_slice, st["base"])

    def plan_g(st):
        bg.prepare_lora_batch(None, st["slots"], st["ranks"], st["scal"], is_decode=True,
                              use_cuda_graph=True)

    plan_g(sets[0])
    side = torch.cuda.Stream(device)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        launch_g(sets[0])
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for st in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            launch_g(st)
        graphs.append(g)
    torch.cuda.synchronize()

    def graph_step(i):
        j = i % len(sets)
        plan_g(sets[j])
        graphs[j].replay()

    gc.collect()
    for i in range(args.warmup):
        graph_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graph_step(i)
    torch.cuda.synchronize()
    graph_wall = time.perf_counter() - t0

    # ---- graph mode with the device planner (secondary): per step, the
    # batch's slot array is copied from pinned host memory into the device
    # buffer the graph reads, then one replay plans on the GPU
    # (lora_plan_device) and runs the embedding gather and the stacked call.
    bd = sgg.ChunkedSgmvLoRA(b0.num_loras, b0.max_chunk_size, device)
    dinfo = bd.init_cuda_graph_batch_info(b0.num_tokens, 1)
    lens_d = torch.ones(b0.num_tokens, dtype=torch.int32, device=device)
    slots_d = torch.zeros(b0.num_tokens, dtype=torch.int32, device=device)
    slots_host = torch.empty((len(sets), b0.num_tokens), dtype=torch.int32, pin_memory=True)
    ws_d = torch.zeros(64 << 20, dtype=torch.uint8, device=device)
    for j, st in enumerate(sets):
        slots_host[j] = torch.from_numpy(st["slots"])
        st["ranks_d"] = torch.from_numpy(st["ranks"]).to(device)
        st["scal_d"] = torch.from_numpy(st["scal"]).to(device)

    def launch_d(st):
        proj = st["proj"]
        bd.prepare_lora_batch_device(lens_d, slots_d, st["ranks_d"], st["scal_d"],
                                     is_decode=True)
        sgg.lora_a_embedding(st["ids"], st["A_emb"], dinfo, vocab, out=st["e"])
        sgg.lora_qkv(st["x"], st["A"], st["B"], dinfo, proj.slice_offsets, proj.max_slice,
                     st["base"], workspace=ws_d)

    slots_d.copy_(slots_host[0])
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        launch_d(sets[0])
    stream.wait_stream(side)
    torch.cuda.synchronize()
    dgraphs = []
    for st in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            launch_d(st)
        dgraphs.append(g)
    torch.cuda.synchronize()

    def dgraph_step(i):
        j = i % len(sets)
        slots_d.copy_(slots_host[j], non_blocking=True)
        dgraphs[j].replay()

    gc.collect()
    for i in range(args.warmup):
        dgraph_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        dgraph_step(i)
    torch.cuda.synchronize()
    dgraph_wall = time.perf_counter() - t0
    # GPU time of the same steps, back to back behind a delay kernel
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    held = hold_stream(stream, 5.0 + 0.2 * args.steps)
    e0.record(stream)
    for i in range(args.steps):
        dgraph_step(i)
    e1.record(stream)
    dgraph_b2b = not held.query()
    torch.cuda.synchronize()
    dgraph_gpu_us = e0.elapsed_time(e1) * 1e3 / args.steps
    del dgraphs

    # host planner alone (native plan into pinned staging + upload), for the record
    t1 = time.perf_counter()
    for i in range(50):
        st = sets[i % len(sets)]
        be.prepare_lora_batch(None, st["slots"], st["ranks"], st["scal"], is_decode=True)
    plan_us = (time.perf_counter() - t1) / 50 * 1e6
    torch.cuda.synchronize()

    hist = seg_histogram(be.prepare_lora_batch(None, sets[0]["slots"], sets[0]["ranks"],
                                               sets[0]["scal"], is_decode=True))
    torch.cuda.synchronize()
    counts = [algo_counts(st["b"], st["proj"], st["A_emb"].shape[1]) for st in sets]
    per = {}
    for n in names:
        avg = dur[n]
        by = float(np.mean([c[n]["bytes"] for c in counts]))
        fl = float(np.mean([c[n]["flops"] for c in counts]))
        per[n] = {"avg_us": round(avg, 3), "algo_bytes": int(by), "algo_flops": int(fl),
                  "gbs": round(by / (avg * 1e-6) / 1e9, 1),
                  "tflops": round(fl / (avg * 1e-6) / 1e12, 3)}
    # the stacked call as the step runs it (two launches), and its one-launch form
    se_us = dur["qkv"]
    se_bytes = per["shrink"]["algo_bytes"] + per["expand"]["algo_bytes"]
    se_flops = per["shrink"]["algo_flops"] + per["expand"]["algo_flops"]
    return {
        "wall_s": eager_wall, "graph_wall_s": graph_wall, "tokens": b0.num_tokens,
        "separate": {"ms_per_step": round(separate_wall / args.steps * 1e3, 4),
                     "tokens_per_s": round(b0.num_tokens * args.steps / separate_wall, 1),
                     "step": "host plan + upload (copy kernel), embedding gather, lora_qkv "
                             "(two launches)"},
        "upload_launch": upload,
        "step_gpu_us": round(step_gpu_us, 2),
        "graph_device_plan": {
            "ms_per_step": round(dgraph_wall / args.steps * 1e3, 4),
            "tokens_per_s": round(b0.num_tokens * args.steps / dgraph_wall, 1),
            "gpu_us_per_step": round(dgraph_gpu_us, 2), "gpu_back_to_back": dgraph_b2b,
            "step": "slot array copied from pinned host memory, then one graph replay: "
                    "lora_plan_device, embedding gather, lora_qkv (two launches)"},
        "priming": {"steps": primed, "ms": round(prime_ms, 1)},
        "kernels": per, "prepare_host_us": round(plan_us, 2), "back_to_back": back_to_back,
        "segment_lengths": hist,
        "shrink_expand": {"us": round(se_us, 3), "algo_bytes": int(se_bytes),
                          "algo_flops": int(se_flops),
                          "gbs": round(se_bytes / (se_us * 1e-6) / 1e9, 1),
                          "hbm_frac": round(se_bytes / (se_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "tokens_per_s_kernels": round(b0.num_tokens / (se_us * 1e-6), 1),
                          "launches": "two (split-K shrink partials, then the expand sums them)",
                          "one_launch_us": round(dur["qkv_one_launch"], 3)},
    }


def run_floor(device, steps=100, sets=48):
    """What the decode kernels' sizes allow on this stack: an empty kernel and
    device-to-device copies whose read + write bytes equal the decode
    shrink's and the stacked call's algorithmic bytes, each launched once per
    step back to back behind a delay kernel (the decode kernels' timing
    protocol), over `sets` rotated buffers so the copies read HBM."""
    import torch
    stream = torch.cuda.current_stream(device)
    out = {}

    def timed(fn):
        for i in range(10):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        held = hold_stream(stream, 5.0 + 0.05 * steps)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        b2b = not held.query()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / steps, 3), b2b

    out["empty_kernel_us"], out["empty_back_to_back"] = timed(lambda i: torch.cuda._sleep(0))
    # host time of one replay of a captured graph holding one empty kernel
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        torch.cuda._sleep(0)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        torch.cuda._sleep(0)
    for _ in range(10):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    host = time.perf_counter() - t0
    torch.cuda.synchronize()
    out["empty_graph_replay_host_us"] = round(host / steps * 1e6, 2)
    del g
    for name, moved in (("shrink", 5268480), ("shrink_expand", 5268480 + 7889920)):
        n = moved // 2
        src = [torch.empty(n, dtype=torch.uint8, device=device) for _ in range(sets)]
        dst = [torch.empty(n, dtype=torch.uint8, device=device) for _ in range(sets)]
        us, b2b = timed(lambda i: dst[i % sets].copy_(src[i % sets]))
        out[f"copy_{name}_bytes"] = moved
        out[f"copy_{name}_us"] = us
        out[f"copy_{name}_gbs"] = round(moved / (us * 1e-6) / 1e9, 1)
        out[f"copy_{name}_back_to_back"] = b2b
        del src, dst
    return out


def _rates(n_bytes, flops, us):
    """GB/s, TFLOP/s and roofline fractions of one call of `us` microseconds.
    fraction_of_attainable = max(bytes / HBM peak, flops / bf16 peak) / time."""
    t = us * 1e-6
    roof = max(n_bytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    return {"avg_us": round(us, 2), "gbs": round(n_bytes / t / 1e9, 1),
            "hbm_frac": round(n_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(flops / t / 1e12, 2),
            "mfma_frac": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4),
            "fraction_of_attainable": round(roof / t, 4)}


def measure_projection(device, b, proj, sets, max_chunk, steps, warmup, emb_rank=16):
    """Events around each call, `steps` times after `warmup`: the shrink, the
    expand and (stacked projections) the stacked call, on one planned batch.
    Call i reads input set i mod len(sets) (`sets`: dicts of device tensors
    x, A, B, base), so repeated calls do not find their inputs in the MALL.
    Also reports the plan's segment-length histogram and the host time of
    the plan + upload call."""
    import torch
    import segmented_gather_gemm_amd as sgg

    be = sgg.ChunkedSgmvLoRA(b.num_loras, max_chunk, device)
    plan_us = host_plan_us(be, b)
    info = be.prepare_lora_batch(None if b.is_decode else b.seq_lens, b.req_slots,
                                 b.lora_ranks, b.scalings, is_decode=b.is_decode)
    c = proj.num_slices
    h = torch.empty((b.num_tokens, sets[0]["A"].shape[1]), dtype=torch.bfloat16, device=device)
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device)
    calls = {
        "shrink": lambda t: sgg.lora_shrink(t["x"], t["A"], info, c, out=h, workspace=ws),
        "expand": lambda t: sgg.lora_expand(h, t["B"], info, proj.slice_offsets, proj.max_slice,
                                            t["base"]),
    }
    if c > 1:
        calls["stacked"] = lambda t: sgg.lora_qkv(t["x"], t["A"], t["B"], info,
                                                  proj.slice_offsets, proj.max_slice, t["base"],
                                                  workspace=ws)
    cnt = algo_counts(b, proj, emb_rank)
    cnt["stacked"] = {k: cnt["shrink"][k] + cnt["expand"][k] for k in ("bytes", "flops")}
    out = {"tokens": b.num_tokens, "segments": info.num_segments,
           "work_segments": info.num_work_segments, "chunk": info.max_len,
           "input_sets": len(sets), "segment_lengths": seg_histogram(info),
           "plan_host_us": plan_us}
    for name, fn in calls.items():
        for i in range(warmup):
            fn(sets[i % len(sets)])
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            fn(sets[i % len(sets)])
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]))
        out[name] = _rates(cnt[name]["bytes"], cnt[name]["flops"], us)
    tot = out["stacked"]["avg_us"] if c > 1 else out["shrink"]["avg_us"] + out["expand"]["avg_us"]
    out["tokens_per_s"] = round(b.num_tokens / (tot * 1e-6), 1)
    return out


def copy_floor_us(device, moved, reps=5):
    """Microseconds of a device-to-device copy moving `moved` bytes (half
    read, half written): what a pure stream of the same bytes takes here."""
    import torch
    n = moved // 2
    src = torch.empty(n, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        dst.copy_(src)
        ev[i + 1].record()
    torch.cuda.synchronize()
    us = float(np.median([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]))
    del src, dst
    torch.cuda.empty_cache()
    return us


def _to(device, d):
    return {k: v.to(device) for k, v in d.items()}


def run_prefill(device, chunks=(16, 32, 64, 128), steps=20, warmup=3):
    """Prefill gate_up (32 requests of 64..2048 tokens, 32 adapters Zipf(1.1),
    r=64, 4096 -> 2 x 14336), one entry per server chunk cap.  One call moves
    4.3 GB, far more than the MALL, so one input set suffices."""
    from synth import draw_batch, draw_projection
    res = {}
    t = None
    for mc in chunks:
        b = draw_batch("prefill", max_chunk_size=mc)
        proj = b.projections[0]
        if t is None:
            t = _to(device, draw_projection(b, proj))
        res[f"chunk{mc}"] = measure_projection(device, b, proj, [t], mc, steps, warmup)
    res["workload"] = ("prefill gate_up, 32 requests (s=%d), 32 adapters Zipf(1.1), r=64, "
                       "4096 -> 2x14336" % b.num_tokens)
    # the shrink's opt-in segment-pair tiles (256 tokens, K in two ranges), for the record
    import segmented_gather_gemm_amd as sgg
    old = sgg.lora_set_option("shrink_pair_tiles", 1)
    try:
        m = measure_projection(device, b, proj, [t], chunks[-1], steps, warmup)
    finally:
        sgg.lora_set_option("shrink_pair_tiles", old)
    res["segment_pair_tiles"] = {"chunk": chunks[-1], "shrink": m["shrink"],
                                 "stacked": m["stacked"]}
    # the expand next to a device copy of its algorithmic bytes
    exp_bytes = algo_counts(b, proj, 16)["expand"]["bytes"]
    del t
    floor = copy_floor_us(device, exp_bytes)
    res["expand_copy_floor"] = {"bytes": int(exp_bytes), "copy_us": round(floor, 1),
                                "copy_gbs": round(exp_bytes / (floor * 1e-6) / 1e9, 1)}
    for mc in chunks:
        r = res[f"chunk{mc}"]["expand"]
        r["fraction_of_copy_floor"] = round(floor / r["avg_us"], 4)
    return res


def run_skewed(device, steps=20, warmup=4, n_sets=4):
    """Skewed mixed batch: 8192 tokens, 90 % on one adapter, ranks 8..64 padded
    to 64 (NaN padding), o_proj 4096 -> 4096 and down_proj 14336 -> 4096;
    `n_sets` rotated input sets (>= 1 GB) so repeated calls read HBM."""
    import torch
    from synth import draw_batch, draw_projection
    b = draw_batch("skewed")
    res = {"workload": "skewed: s=8192, 128 adapters, 90 % on one, ranks {8,16,32,64} "
                       "padded to 64"}
    for pi, proj in enumerate(b.projections):
        sets = rotated(_to(device, draw_projection(b, proj, proj_index=pi)), n_sets)
        res[proj.name] = measure_projection(device, b, proj, sets, b.max_chunk_size, steps,
                                            warmup)
        del sets
        torch.cuda.empty_cache()
    return res


def run_decode_sizes(device, sizes=(1024, 2048, 4096, 16384), steps=20, warmup=4, n_sets=3):
    """The decode batch's shape at more requests: n one-token requests on 8
    adapters drawn uniformly, rank 16, stacked qkv 4096 -> [4096, 1024, 1024];
    shrink, expand and the stacked call with their HBM fractions, to show
    where the kernels leave the launch-and-latency regime of 256 tokens."""
    import torch
    from synth.workloads import Batch, Projection
    from synth import draw_projection
    res = {"workload": "decode-shaped batches: n x 1 token, 8 adapters uniform, r=16, "
                       "stacked qkv 4096 -> [4096,1024,1024]"}
    for n in sizes:
        rng = np.random.default_rng(1002 + n)
        b = Batch(f"decode_{n}", 1002 + n, [1] * n, rng.integers(0, 8, n).tolist(), True, 8,
                  [16] * 8, [1.0] * 8, 128, [Projection("qkv", 4096, [0, 4096, 5120, 6144], 16)])
        proj = b.projections[0]
        sets = rotated(_to(device, draw_projection(b, proj)), n_sets)
        res[str(n)] = measure_projection(device, b, proj, sets, 128, steps, warmup)
        del sets
        torch.cuda.empty_cache()
    return res


def run_full(device, layers, steps=5, warmup=1):
    """Full layer sweep, Llama-3-8B shapes: per layer qkv, o, gate_up, down
    over 4288 tokens (192 decode + 8 x 512), 64 adapters r=32, one plan.
    `layers` layers with distinct weights and activations (~0.9 GB each) are
    resident and run in sequence, as a forward pass does, so no call finds its
    inputs in the MALL; each call is timed with events around it.  Stacked
    projections run as the stacked call (their standalone shrink and expand
    are timed in a second sweep); the per-layer figure is the mean over layers
    and passes, and the 32-layer figure is 32 x that."""
    import torch
    from synth import draw_batch, draw_embedding, draw_projection
    import segmented_gather_gemm_amd as sgg
    b = draw_batch("full")
    be = sgg.ChunkedSgmvLoRA(b.num_loras, b.max_chunk_size, device)
    plan_us = host_plan_us(be, b)
    info = be.prepare_lora_batch(b.seq_lens, b.req_slots, b.lora_ranks, b.scalings)
    hist = seg_histogram(info)
    projs = b.projections
    data = [[_to(device, draw_projection(b, p, layer=layer, proj_index=pi))
             for pi, p in enumerate(projs)] for layer in range(layers)]
    hs = [torch.empty((b.num_tokens, t["A"].shape[1]), dtype=torch.bfloat16, device=device)
          for t in data[0]]
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device)

    def call(kind, pi, t):
        p = projs[pi]
        if kind == "stacked":
            sgg.lora_qkv(t["x"], t["A"], t["B"], info, p.slice_offsets, p.max_slice, t["base"],
                         workspace=ws)
        elif kind == "shrink":
            sgg.lora_shrink(t["x"], t["A"], info, p.num_slices, out=hs[pi], workspace=ws)
        else:
            sgg.lora_expand(hs[pi], t["B"], info, p.slice_offsets, p.max_slice, t["base"])

    def sweep(kinds_of):
        """Events around every call of `warmup + steps` passes over the layers;
        mean microseconds per (projection, kind) over the timed passes."""
        times = {}
        for rep in range(warmup + steps):
            evs = []
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            for layer in range(layers):
                for pi in range(len(projs)):
                    for kind in kinds_of(pi):
                        call(kind, pi, data[layer][pi])
                        e2 = torch.cuda.Event(enable_timing=True)
                        e2.record(stream)
                        evs.append((pi, kind, e, e2))
                        e = e2
            torch.cuda.synchronize()
            if rep >= warmup:
                for pi, kind, a, z in evs:
                    times.setdefault((pi, kind), []).append(a.elapsed_time(z) * 1e3)
        return {k: float(np.mean(v)) for k, v in times.items()}

    main = sweep(lambda pi: ("stacked",) if projs[pi].num_slices > 1 else ("shrink", "expand"))
    parts = sweep(lambda pi: ("shrink", "expand"))
    per = {}
    per_kernels = {}
    for pi, p in enumerate(projs):
        per[p.name] = (main[(pi, "stacked")] if p.num_slices > 1 else
                       main[(pi, "shrink")] + main[(pi, "expand")])
        per_kernels[p.name] = {k: round(parts[(pi, k)], 2) for k in ("shrink", "expand")}
    layer_us = float(sum(per.values()))
    cnts = [algo_counts(b, p, 16) for p in projs]
    layer_bytes = sum(c["shrink"]["bytes"] + c["expand"]["bytes"] for c in cnts)
    layer_flops = sum(c["shrink"]["flops"] + c["expand"]["flops"] for c in cnts)
    per_proj = {}
    for pi, p in enumerate(projs):
        cb = cnts[pi]["shrink"]["bytes"] + cnts[pi]["expand"]["bytes"]
        cf = cnts[pi]["shrink"]["flops"] + cnts[pi]["expand"]["flops"]
        per_proj[p.name] = _rates(cb, cf, per[p.name])
    del data
    torch.cuda.empty_cache()
    # embedding gather over the same plan (A_emb is 263 MB, above the MALL)
    ids, A_emb = draw_embedding(b)
    ids, A_emb = ids.to(device), A_emb.to(device)
    e_out = torch.empty((b.num_tokens, A_emb.shape[1]), dtype=torch.bfloat16, device=device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sgg.lora_a_embedding(ids, A_emb, info, b.vocab_size, out=e_out)
    e0.record(stream)
    for _ in range(20):
        sgg.lora_a_embedding(ids, A_emb, info, b.vocab_size, out=e_out)
    e1.record(stream)
    torch.cuda.synchronize()
    emb_us = e0.elapsed_time(e1) * 1e3 / 20
    emb_bytes = algo_counts(b, projs[0], A_emb.shape[1])["embedding"]["bytes"]
    return {"workload": "full layer sweep: Llama-3-8B shapes, 4288 tokens, 64 adapters r=32; "
                        f"{layers} resident layers with distinct weights and activations, "
                        f"{steps} timed passes",
            "segments": info.num_segments, "work_segments": info.num_work_segments,
            "segment_lengths": hist, "plan_host_us": plan_us,
            "per_layer_us": {k: round(v, 2) for k, v in per.items()},
            "per_projection": per_proj,
            "per_layer_kernels_us": per_kernels,
            "layer": _rates(layer_bytes, layer_flops, layer_us),
            "layers32_ms": round(32 * layer_us / 1e3, 3),
            "tokens_per_s_32_layers": round(b.num_tokens / (32 * layer_us * 1e-6), 1),
            "embedding": {"avg_us": round(emb_us, 2), "algo_bytes": int(emb_bytes),
                          "gbs": round(emb_bytes / (emb_us * 1e-6) / 1e9, 2)}}


def run_lm_head(device, steps=20, warmup=3):
    """Pruned lm_head pass of the decode batch: each of the 256 requests sends
    one token to the lm_head (4096 -> vocab 128256, r=16, 8 adapters).  The
    lm_head plan keeps the tokens in original order (identity permutation), so
    its segments are runs of consecutive same-slot requests -- about one token
    each when the adapters are dealt uniformly.  The sorted plan of the same
    tokens is timed beside it."""
    import torch
    import segmented_gather_gemm_amd as sgg
    from synth import draw_batch, draw_projection
    from synth.workloads import Projection
    b = draw_batch("decode")
    proj = Projection("lm_head", 4096, [0, 128256], 16)
    # about 100 MB per call: 4 rotated input sets keep repeated calls off the MALL
    sets = rotated(_to(device, draw_projection(b, proj, proj_index=len(b.projections))), 4)
    cnt = algo_counts(b, proj, 16)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=device)
    h = torch.empty((b.num_tokens, proj.rank), dtype=torch.bfloat16, device=device)
    stream = torch.cuda.current_stream(device)
    res = {"workload": "lm_head pass of the decode batch: 256 requests x 1 token, 8 adapters "
                       "uniform, r=16, 4096 -> 128256"}
    for mode in ("identity_plan", "sorted_plan"):
        be = sgg.ChunkedSgmvLoRA(b.num_loras, b.max_chunk_size, device)
        if mode == "identity_plan":
            info = be.prepare_lm_head_batch([1] * len(b.req_slots), b.req_slots, b.lora_ranks,
                                            b.scalings)
        else:
            info = be.prepare_lora_batch(None, b.req_slots, b.lora_ranks, b.scalings,
                                         is_decode=True)
        calls = {
            "shrink": lambda t: sgg.lora_shrink(t["x"], t["A"], info, 1, out=h, workspace=ws),
            "expand": lambda t: sgg.lora_expand(h, t["B"], info, proj.slice_offsets,
                                                proj.max_slice, t["base"]),
        }
        out = {"segments": info.num_segments, "work_segments": info.num_work_segments,
               "segment_lengths": seg_histogram(info)}
        for name, fn in calls.items():
            for i in range(warmup):
                fn(sets[i % len(sets)])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                fn(sets[i % len(sets)])
            e1.record(stream)
            torch.cuda.synchronize()
            out[name] = _rates(cnt[name]["bytes"], cnt[name]["flops"],
                               e0.elapsed_time(e1) * 1e3 / steps)
        tot = out["shrink"]["avg_us"] + out["expand"]["avg_us"]
        out["tokens_per_s"] = round(b.num_tokens / (tot * 1e-6), 1)
        res[mode] = out
    return res


def run_short_segments(device, steps=50, warmup=5, n_sets=8):
    """The shrink's two arithmetic forms on batches of short segments: MFMA
    tiles (default) and the VALU form (library option shrink_valu: 16-token
    tiles, those with at most 4 tokens summed on the VALU with cross-lane
    reductions).  Batches: 256 one-token decode requests over 128 adapters
    (segments of ~2 tokens; stacked qkv, r=16) and the full-layer batch's
    o_proj (192 one-token requests + 8 x 512 over 64 adapters, r=32)."""
    import segmented_gather_gemm_amd as sgg
    from synth import draw_batch, draw_projection
    from synth.workloads import Batch, Projection
    rng = np.random.default_rng(20261203)
    many = Batch("decode_128_adapters", 20261203, [1] * 256,
                 rng.integers(0, 128, 256).tolist(), True, 128, [16] * 128, [1.0] * 128, 128,
                 [Projection("qkv", 4096, [0, 4096, 5120, 6144], 16)])
    full = draw_batch("full")
    o_proj = [p for p in full.projections if p.in_dim == 4096 and p.num_slices == 1][0]
    res = {"workload": "short segments: decode 256 x 1 token over 128 adapters (qkv c=3, r=16); "
                       "full-layer batch o_proj 4096 -> 4096 (r=32)"}
    for name, b, proj in (("decode_128_adapters", many, many.projections[0]),
                          ("full_o_proj", full, o_proj)):
        sets = rotated(_to(device, draw_projection(b, proj)), n_sets)
        out = {}
        for form, flag in (("mfma", 0), ("valu", 1)):
            old = sgg.lora_set_option("shrink_valu", flag)
            try:
                m = measure_projection(device, b, proj, sets, b.max_chunk_size, steps, warmup)
            finally:
                sgg.lora_set_option("shrink_valu", old)
            out[form] = {k: m[k] for k in ("shrink", "stacked") if k in m}
            out["segment_lengths"] = m["segment_lengths"]
            out["segments"] = m["segments"]
        res[name] = out
        del sets
    return res


def run_moe(device, steps=50, warmup=5, n_sets=8):
    """MoE LoRA add on a decode batch (256 one-token requests, 8 adapters,
    r=16) routed top-2 over 8 experts, LoRA on the experts' up projection
    (4096 -> 14336): per step, the routing and the copies' plan on the GPU
    in one launch (lora_moe_plan) and lora_moe_add into the fused-MoE
    intermediate (512 rows); the routing and the plan as two launches
    (lora_moe_route, then lora_plan_device) are timed beside them.  HIP
    events around each call, back to back."""
    import torch
    import segmented_gather_gemm_amd as sgg
    rng = np.random.default_rng(20261204)
    s, L, E, k, K, N, R = 256, 8, 8, 2, 4096, 14336, 16
    slots = rng.integers(0, L, s).tolist()
    ranks, scal = [R] * L, [1.0] * L
    be = sgg.ChunkedSgmvLoRA(L, 128, device)
    be.prepare_lora_batch(None, slots, ranks, scal, is_decode=True)
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(device)
    sets = []
    for i in range(n_sets):
        topk = np.stack([rng.permutation(E)[:k] for _ in range(s)]).astype(np.int32)
        sets.append({"topk": torch.from_numpy(topk).to(device),
                     "x": bf(rng.standard_normal((s, K))),
                     "A": bf(rng.standard_normal((L, E, R, K)) * 0.02),
                     "B": bf(rng.standard_normal((L, E, N, R)) * 0.02),
                     "out": bf(rng.standard_normal((s * k, N)))})
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device)
    infos = {}

    def plan(i):
        infos[i % n_sets] = be.prepare_moe_lora_batch(sets[i % n_sets]["topk"], E)

    def add(i):
        st = sets[i % n_sets]
        sgg.lora_moe_add(st["x"], st["A"], st["B"], be.moe_batch_info, k, st["out"],
                         workspace=ws)

    # the same routing and plan as two launches, into buffers of their own
    nv, copies = L * E + 1, s * k
    seg_cap = sgg.lora_plan_max_segments(copies, nv, 16)
    offs = (ctypes.c_int64 * 10)()
    total = int(sgg.lib().lora_plan_layout(copies, seg_cap, copies, nv, offs))
    two = {"slots": torch.zeros(copies, dtype=torch.int32, device=device),
           "vranks": torch.zeros(nv, dtype=torch.int32, device=device),
           "vscal": torch.zeros(nv, dtype=torch.float32, device=device),
           "plan": torch.zeros(total, dtype=torch.int32, device=device),
           "info": torch.zeros(8, dtype=torch.int32, device=device)}

    def route_then_plan(i):
        bi = be.batch_info
        sgg.lora_moe_route(bi.req_seg_indptr, bi.req_weight_indices, bi.bs,
                           sets[i % n_sets]["topk"], E, bi.lora_ranks, bi.scalings, L,
                           two["slots"], two["vranks"], two["vscal"])
        sgg.lora_plan_device(None, two["slots"], two["vranks"], two["vscal"], nv, True, 128, 0,
                             copies, seg_cap, copies, two["plan"], two["info"])

    res = {"workload": f"MoE LoRA add: decode {s} x 1 token, {L} adapters r={R}, top-{k} of "
                       f"{E} experts, expert up projection {K} -> {N}; {s * k} copies over "
                       f"{L * E} virtual experts", "input_sets": n_sets}
    for name, fn in (("route_and_plan", plan), ("route_then_plan_two_launches", route_then_plan),
                     ("plan_then_add", None)):
        if fn is None:
            def fn(i):
                plan(i)
                add(i)
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        held = hold_stream(stream, 5.0 + 0.1 * steps)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        b2b = not held.query()
        torch.cuda.synchronize()
        res[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
        res[name + "_back_to_back"] = b2b
    add_us = res["plan_then_add_us"] - res["route_and_plan_us"]
    # algorithmic bytes of the add: x once, each active virtual expert's A and
    # B once, the intermediate rows read and written once
    act = len({(a, int(e)) for st in sets[:1] for a, row in zip(slots, st["topk"].cpu().numpy())
               for e in row})
    by = 2 * s * K + act * R * (K + N) * 2 + 2 * 2 * s * k * N
    res["add_us"] = round(add_us, 2)
    res["add_algo_bytes"] = int(by)
    res["add_gbs"] = round(by / (add_us * 1e-6) / 1e9, 1)
    res["add_hbm_frac"] = round(by / (add_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    res["tokens_per_s"] = round(s / (res["plan_then_add_us"] * 1e-6), 1)
    return res


def run_device_plan(device, steps=200):
    """The device-side planner (lora_plan_device) on the decode batch and on
    the prefill batch, one launch per step back to back behind a delay
    kernel; the host planner with its upload timed the same way beside it."""
    import torch
    import segmented_gather_gemm_amd as sgg
    from synth import draw_batch
    stream = torch.cuda.current_stream(device)
    res = {}
    for name, b in (("decode", draw_batch("decode")), ("prefill", draw_batch("prefill"))):
        decode = b.is_decode
        max_bs = len(b.req_slots)
        tpb = 1 if decode else max(b.seq_lens)
        be = sgg.ChunkedSgmvLoRA(b.num_loras, b.max_chunk_size, device)
        be.init_cuda_graph_batch_info(max_bs, tpb)
        i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=device)
        lens_d = i32(b.seq_lens)
        slots_d, ranks_d = i32(b.req_slots), i32(b.lora_ranks)
        scal_d = torch.tensor(b.scalings, dtype=torch.float32, device=device)
        slots, ranks = np.asarray(b.req_slots, np.int32), np.asarray(b.lora_ranks, np.int32)
        scal = np.asarray(b.scalings, np.float32)
        lens = None if decode else np.asarray(b.seq_lens, np.int32)
        calls = {
            "device_planner_us": lambda: be.prepare_lora_batch_device(
                lens_d, slots_d, ranks_d, scal_d, is_decode=decode),
            "host_planner_and_upload_us": lambda: be.prepare_lora_batch(
                lens, slots, ranks, scal, is_decode=decode, use_cuda_graph=True),
        }
        out = {"tokens": b.num_tokens, "requests": max_bs}
        for key, fn in calls.items():
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            held = hold_stream(stream, 5.0 + 0.05 * steps)
            e0.record(stream)
            for _ in range(steps):
                fn()
            e1.record(stream)
            b2b = not held.query()
            torch.cuda.synchronize()
            out[key] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
            out[key.replace("_us", "_back_to_back")] = b2b
        res[name] = out
    return res


def fused_timeline(device, calls=40):
    """Per-workgroup timeline of the one-launch stacked call on the decode
    batch: each call runs alone (synchronised before and after) and its
    workgroups' start, wait-done and end times are read back; the figures are
    medians over the calls of each call's percentiles, in microseconds from
    the call's first workgroup start."""
    import torch
    import segmented_gather_gemm_amd as sgg
    sets = make_sets(8, device)
    b0 = sets[0]["b"]
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=device)
    be = sgg.ChunkedSgmvLoRA(b0.num_loras, b0.max_chunk_size, device)
    infos = [own_plan(be.prepare_lora_batch(None, np.asarray(st["b"].req_slots, np.int32),
                                            np.asarray(st["b"].lora_ranks, np.int32),
                                            np.asarray(st["b"].scalings, np.float32),
                                            is_decode=True)) for st in sets]
    cap = 1 << 16
    trace = torch.zeros(4 * cap, dtype=torch.int64, device=device)

    def call(i):
        st, info = sets[i % len(sets)], infos[i % len(sets)]
        p = st["proj"]
        sgg.lora_qkv(st["x"], st["A"], st["B"], info, p.slice_offsets, p.max_slice, st["base"],
                     workspace=ws)

    old = {"fused_stacked": sgg.lora_set_option("fused_stacked", 1)}
    for i in range(10):
        call(i)
    torch.cuda.synchronize()
    old["fused_trace_blocks"] = sgg.lora_set_option("fused_trace_blocks", cap)
    old["fused_trace"] = sgg.lora_set_option("fused_trace", trace.data_ptr())
    pct = (0, 10, 50, 90, 100)
    rows = []
    try:
        for i in range(calls):
            trace.zero_()
            torch.cuda.synchronize()
            call(i)
            torch.cuda.synchronize()
            t = trace.view(-1, 4).cpu().numpy().astype(np.int64)
            t = t[t[:, 0] > 0]
            base = t[:, 0].min()
            us = lambda a: [round(float(np.percentile(a, q)) * 0.01, 2) for q in pct]
            prod, cons = t[t[:, 3] == 0], t[t[:, 3] >= 1]
            waited = cons[cons[:, 1] > 0]
            rows.append({
                "span": [round((t[:, 2].max() - base) * 0.01, 2)],
                "shrink_tile_start": us(prod[:, 0] - base),
                "shrink_tile_work_done": us(prod[:, 1] - base),
                "shrink_tile_busy": us(prod[:, 1] - prod[:, 0]),
                "expand_tile_start": us(cons[:, 0] - base),
                "expand_tile_wait_done": us(waited[:, 1] - base),
                "expand_tile_end": us(cons[:, 2] - base),
                "expand_tile_after_wait": us(waited[:, 2] - waited[:, 1]),
                "counts": [len(prod), len(cons), int((cons[:, 3] == 2).sum())]})
    finally:
        for k, v in old.items():
            sgg.lora_set_option(k, v)
    out = {"workload": "decode: 256 requests x 1 token, 8 adapters, r=16, stacked qkv "
                       "4096 -> [4096,1024,1024]", "calls": calls,
           "percentiles": list(pct), "unit": "us from the call's first workgroup start"}
    for k in rows[0]:
        if k == "counts":
            continue
        out[k] = [round(float(np.median([r[k][j] for r in rows])), 2)
                  for j in range(len(rows[0][k]))]
    c = rows[-1]["counts"]
    out["workgroups"] = {"shrink_tiles": c[0], "expand_tiles": c[1],
                         "gave_up_waiting": max(r["counts"][2] for r in rows)}
    print(json.dumps(out), flush=True)


def copy_probe(device):
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=device)
    bb = torch.empty_like(a)
    for _ in range(5):
        bb.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}))


# ----------------------------------------------------------------- CPU leg

def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(seconds):
    """The oracle (plan oracle + fp64 math oracle) on the decode workload's
    rotated batches until `seconds` have elapsed, with BLAS allowed every core
    this process may run on."""
    from threadpoolctl import threadpool_limits
    from oracle import lora as ol
    from oracle import plan as op
    from synth import draw_batch, draw_embedding, draw_projection, to_f64
    from synth.workloads import rotation_batch

    cores = len(os.sched_getaffinity(0))
    base_b = draw_batch("decode")
    prepared = []
    for i in range(2):
        b = base_b if i == 0 else rotation_batch(base_b, i)
        proj = b.projections[0]
        t = draw_projection(b, proj)
        ids, A_emb = draw_embedding(b)
        prepared.append((b, proj, {k: to_f64(v) for k, v in t.items()}, ids.numpy(),
                         to_f64(A_emb)))
    done = 0
    tokens = 0
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        while True:
            b, proj, t, ids, A_emb = prepared[done % len(prepared)]
            op.plan(None, b.req_slots, True, b.max_chunk_size)
            ol.lora_forward(t["x"], t["A"], t["B"], t["base"], b.seq_lens, b.req_slots,
                            b.lora_ranks, b.scalings, proj.slice_offsets)
            ol.embedding_a(ids, A_emb, b.seq_lens, b.req_slots, b.lora_ranks, 128256)
            done += 1
            tokens += b.num_tokens
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": round(tokens / el, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} full decode steps (256 tokens each: plan + qkv shrink/expand + "
                      f"embedding gather, fp64 NumPy), {el:.1f} s, BLAS threads = {cores} "
                      f"(the process's CPU affinity)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is "
              f"single-GPU, with no sharding or collectives", file=sys.stderr)
        sys.exit(2)
    bad = [x for x in args.legs.split(",") if x and x not in LEGS]
    if bad:
        print(f"unknown legs {bad}; known: {', '.join(LEGS)}", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(device)
        return
    if args.fused_timeline:
        fused_timeline(device)
        return
    print(f"# decode: {args.sets} input sets, warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    res = run_decode(args, device)
    ms = res["wall_s"] / args.steps * 1e3
    value = res["tokens"] * args.steps / res["wall_s"]
    graph = res["tokens"] * args.steps / res["graph_wall_s"]
    k = res["kernels"]
    se = res["shrink_expand"]
    # the longest of the step's kernels (timed standalone) is the dominant one
    dom_name = max(("shrink", "expand", "embedding"), key=lambda n: k[n]["avg_us"])
    dom = {"us": k[dom_name]["avg_us"], "gbs": k[dom_name]["gbs"]}
    achieved = dom["gbs"]
    line = {
        "metric": "LoRA tokens/s (decode qkv shrink+expand + embedding gather, whole step)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode: 256 requests x 1 token, 8 adapters uniform, r=16, "
                               "stacked qkv 4096 -> [4096,1024,1024] (c=3), chunk cap 128; "
                               "LoRA-A embedding vocab 128256 r=16; "
                               f"{args.sets} rotated input sets",
                   "tokens_per_step": res["tokens"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(dom_name, "decode"),
                     "algo_bytes_per_launch": k[dom_name]["algo_bytes"],
                     "avg_launch_us": dom["us"]},
        "mode": "eager: host plan, then one launch that uploads the plan and does the "
                "embedding gather, then lora_qkv (two launches)",
        "separate_upload_and_embedding": res["separate"],
        "upload_launch": res["upload_launch"],
        "step_gpu_us": res["step_gpu_us"],
        "graph_tokens_per_s": round(graph, 1),
        "graph_ms_per_step": round(res["graph_wall_s"] / args.steps * 1e3, 4),
        "graph_device_plan": res["graph_device_plan"],
        "kernels": k,
        "kernel_timing": ("HIP events on the launch stream around one launch per step, "
                          "back to back behind a delay kernel" + ("" if res["back_to_back"] else
                                            " (WARNING: delay ended before enqueueing did)")),
        "shrink_expand": res["shrink_expand"],
        "prepare_host_us": res["prepare_host_us"],
        "segment_lengths": res["segment_lengths"],
        "priming": res["priming"],
    }
    print("# floor", file=sys.stderr, flush=True)
    floor = run_floor(device)
    line["floor"] = floor
    # fraction of what the sizes allow: the same bytes moved by a device copy
    line["kernels"]["shrink"]["fraction_of_copy_floor"] = round(
        floor["copy_shrink_us"] / k["shrink"]["avg_us"], 4)
    line["shrink_expand"]["fraction_of_copy_floor"] = round(
        floor["copy_shrink_expand_us"] / res["shrink_expand"]["us"], 4)
    legs = [] if args.quick else [x for x in args.legs.split(",") if x]
    runners = {"prefill": ("prefill chunk sweep", lambda: run_prefill(device)),
               "skewed": ("skewed", lambda: run_skewed(device)),
               "full": ("full layer sweep", lambda: run_full(device, args.full_layers)),
               "lm_head": ("lm_head pass", lambda: run_lm_head(device)),
               "device_plan": ("device planner", lambda: run_device_plan(device)),
               "short": ("short segments: MFMA and VALU shrink",
                         lambda: run_short_segments(device)),
               "moe": ("MoE LoRA add", lambda: run_moe(device)),
               "decode_sizes": ("decode-shaped batches of 1024-16384 tokens",
                                lambda: run_decode_sizes(device))}
    for leg in legs:
        print(f"# {runners[leg][0]}", file=sys.stderr, flush=True)
        line[leg] = runners[leg][1]()
    if not args.no_cpu:
        print("# cpu baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
