"""ChunkedSgmvLoRA: the chunked SGMV LoRA backend API over the C ABI.

Method names and arguments follow the ``ChunkedSgmvLoRABackend`` /
``BaseLoRABackend`` pages (prepare_lora_batch, run_lora_a_sgemm,
run_lora_b_sgemm, run_qkv_lora, run_gate_up_lora, run_lora_a_embedding,
init_cuda_graph_batch_info); the pruned lm_head plans of
``_prepare_lm_head_batch_info`` are prepare_lm_head_batch and
prepare_lm_head_pass_batches.  Every step of the work runs in libsgg_lora:
the plan in its host planner, the rest in its HIP kernels.

Upload: the page copies six small host arrays to the device one by one.
Here one native call (lora_plan_upload) plans straight into a pinned staging
buffer and enqueues a single non-blocking host-to-device transfer of all plan
arrays and tables; the device arrays are views of one device buffer.  Plan
buffers (staging + device) rotate through a ring of 8 slots; a slot is reused
only after the transfer that last read it has completed, so planning the next
batch does not wait for the GPU.  A batch's device plan stays intact while
fewer than 8 further batches have been prepared, or for as long as its
kernels run on the stream it was prepared on (later uploads are ordered
after them).
"""

import ctypes
import time

import numpy as np
import torch

from . import binding as B
from ._lib import calls, check, lib
from .binding import LoRABatchInfo

_P32 = ctypes.POINTER(ctypes.c_int32)

MIN_CHUNK_SIZE = 16


def _align(n, m=64):
    return (n + m - 1) // m * m


def batch_arrays(seq_lens, weight_indices, lora_ranks, scalings, max_loras):
    """Host arrays of one batch, checked before the native planner reads them:
    (lens or None, slots, ranks, scalings, tokens).

    ``seq_lens`` None means decode mode (one token per request); otherwise it
    needs one entry per entry of ``weight_indices`` -- the planner reads
    ``seq_lens[r]`` for every request r.  ``lora_ranks`` and ``scalings`` need
    ``max_loras`` entries each.
    """
    if len(lora_ranks) != max_loras or len(scalings) != max_loras:
        raise ValueError(f"lora_ranks and scalings need {max_loras} entries")
    slots = np.ascontiguousarray(weight_indices, dtype=np.int32)
    if slots.ndim != 1:
        raise ValueError("weight_indices must be one-dimensional")
    if seq_lens is None:
        lens, s = None, len(slots)
    else:
        lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        if lens.shape != slots.shape:
            raise ValueError(f"seq_lens has {lens.size} entries, weight_indices {slots.size}")
        s = int(lens.sum(dtype=np.int64))
    ranks = np.ascontiguousarray(lora_ranks, dtype=np.int32)
    scal = np.ascontiguousarray(scalings, dtype=np.float32)
    return lens, slots, ranks, scal, s


class _Staging:
    """Ring of plan buffers: pinned host staging plus a device plan buffer per
    slot.

    Every slot is allocated when the ring is made, and a larger plan grows all
    slots at once, so after the first batch of a given size no batch
    allocates (a pinned allocation costs hundreds of microseconds).  The
    per-slot ``LoRABatchInfo`` views of a plan layout are likewise built for
    all slots the first time that layout is seen.

    A slot's staging buffer is reused only after the upload that last read it
    has done so: the upload's copy kernel writes the slot's sequence number
    into a pinned flag word once it has read the staging buffer, and taking
    the slot polls that word in host memory (no event, no driver call: a
    sleeping wait wakes up tens of microseconds late, which a serving loop
    that plans each batch while the previous one runs cannot afford).  The
    slot's device buffer is then rewritten by an upload enqueued after every
    kernel launched before it on the same stream, so the kernels of a batch
    read its plan intact as long as they run on the stream the batch was
    prepared on.  Buffers outgrown by a larger plan are kept alive, never
    freed: kernels already enqueued may still read them.
    """

    def __init__(self, device, slots=8, words=16384):
        self.device = device
        self.n = slots
        self.host = [None] * slots
        self.dev = [None] * slots
        self.infos = [{} for _ in range(slots)]   # layout key -> LoRABatchInfo views
        self.host_addr = [0] * slots               # staging / device addresses and bytes
        self.dev_addr = [0] * slots
        self.dev_bytes = [0] * slots
        self.retired = []
        self.flags = torch.zeros(slots, dtype=torch.int32, pin_memory=True)
        self.flag_view = self.flags.numpy()
        self.flag_addr = self.flags.data_ptr()
        self.seq = [0] * slots
        self.words = 0
        self.i = 0
        self._grow(words)

    def _grow(self, n):
        """Give every slot a buffer of at least n words (waits for every
        enqueued upload to have read its staging buffer first)."""
        size = max(int(n), 2 * self.words, 4096)
        for i in range(self.n):
            if self.flag_view[i] != self.seq[i]:
                self._wait(i, self.seq[i])
        for i in range(self.n):
            if self.host[i] is not None:
                self.retired.append((self.host[i], self.dev[i]))
            self.host[i] = torch.empty(size, dtype=torch.int32, pin_memory=True)
            self.dev[i] = torch.empty(size, dtype=torch.int32, device=self.device)
            self.host_addr[i] = self.host[i].data_ptr()
            self.dev_addr[i] = self.dev[i].data_ptr()
            self.dev_bytes[i] = 4 * size
            self.infos[i] = {}
        self.words = size

    def take(self, n):
        if n > self.words:
            self._grow(n)
        i = self.i
        self.i = (i + 1) % self.n
        want = self.seq[i]
        if self.flag_view[i] != want:
            self._wait(i, want)
        return i

    def _wait(self, i, want, limit_s=30.0):
        """Poll slot i's flag; raise if the upload has not read its staging
        buffer within `limit_s` seconds (its stream never ran it)."""
        flags = self.flag_view
        t0 = time.monotonic()
        n = 0
        while flags[i] != want:
            n += 1
            if n % 4096 == 0 and time.monotonic() - t0 > limit_s:
                raise RuntimeError(
                    f"plan staging slot {i}: the upload enqueued {limit_s:.0f} s ago has not "
                    "run (is its stream blocked?)")

    def signal(self, i):
        """Flag address and value that the next upload from slot i writes."""
        return self.flag_addr + 4 * i, (self.seq[i] + 1) & 0x7FFFFFFF

    def done(self, i):
        """The upload from slot i was enqueued: wait for its flag next time."""
        self.seq[i] = (self.seq[i] + 1) & 0x7FFFFFFF


_NAMES = ("permutation", "seg_indptr", "seg_slots", "req_seg_indptr", "req_slots", "ranks",
          "scalings", "work_indptr", "work_slots", "work_perm")


class ChunkedSgmvLoRA:
    """Chunked segmented-gather LoRA backend for one device."""

    name = "csgmv"

    def __init__(self, max_loras_per_batch, max_chunk_size=128, device="cuda"):
        self.max_loras_per_batch = int(max_loras_per_batch)
        self.max_chunk_size = int(max_chunk_size)
        self.device = torch.device(device)
        self.batch_info = None
        self.lm_head_batch_info = None
        self.lm_head_pass_batch_infos = None
        self.cuda_graph_batch_info = None
        self._graph_dev = None
        self._graph_cap = None
        self._graph_info_dev = None
        self.cuda_graph_plan_info = None
        self._staging = _Staging(self.device)
        self._layouts = {}
        self._info_arr = (ctypes.c_int32 * 6)()
        self._info_addr = ctypes.addressof(self._info_arr)
        self._info_np = np.frombuffer(self._info_arr, dtype=np.int32)
        self._seg_caps = {}
        self._dev_index = self.device.index
        self._moe = {}
        self.moe_batch_info = None
        self.moe_plan_info = None

    # ---------------------------------------------------------------- plan
    def _layout(self, s_cap, seg_cap, req_cap):
        key = (s_cap, seg_cap, req_cap)
        lay = self._layouts.get(key)
        if lay is None:
            offs = (ctypes.c_int64 * len(_NAMES))()
            total = int(lib().lora_plan_layout(s_cap, seg_cap, req_cap, self.max_loras_per_batch,
                                               offs))
            sizes = (s_cap, seg_cap + 1, seg_cap, req_cap + 1, req_cap,
                     self.max_loras_per_batch, self.max_loras_per_batch, seg_cap + 1, seg_cap,
                     s_cap)
            lay = (total, [(int(o), n) for o, n in zip(offs, sizes)])
            self._layouts[key] = lay
        return lay

    def prepare_lora_batch(self, seq_lens, weight_indices, lora_ranks, scalings,
                           is_decode=False, use_cuda_graph=False, chunk_size_override=0):
        """Plan the batch on the host and upload it with one async copy.

        seq_lens: tokens per request (None in decode mode: one each);
        weight_indices: slot per request; lora_ranks / scalings: per slot
        (``max_loras_per_batch`` entries, rank 0 = no adapter).
        """
        return self._prepare(seq_lens, weight_indices, lora_ranks, scalings, is_decode,
                             use_cuda_graph, chunk_size_override, None)

    def prepare_lora_batch_with_embedding(self, seq_lens, weight_indices, lora_ranks, scalings,
                                          input_ids, weights, vocab_size, is_decode=False,
                                          use_cuda_graph=False, chunk_size_override=0,
                                          out=None):
        """prepare_lora_batch, then run_lora_a_embedding(input_ids, weights,
        vocab_size) over that batch -- the first LoRA call of a forward pass
        -- with the same results.  For decode-shaped batches (one token per
        request) the upload and the lookup are one launch.  Returns
        (batch_info, embedding output of shape (num_tokens, R))."""
        if input_ids.dtype is not torch.int64 or not input_ids.is_cuda:
            raise TypeError("input_ids must be an int64 tensor on a ROCm device")
        B._need_bf16_dense("weights", weights, 3)
        L, R, V = weights.shape
        if L != self.max_loras_per_batch:
            raise ValueError(f"weights hold {L} slots, the backend {self.max_loras_per_batch}")
        ids = input_ids.contiguous()
        s = ids.shape[0]
        if out is None:
            out = torch.empty((s, R), dtype=torch.bfloat16, device=weights.device)
        ost = B._need_bf16("out", out, 2)
        B._need_rows_cols("out", out, s, R)
        emb = (s, ids.data_ptr(), weights.data_ptr(), V, out.data_ptr(), ost[0], R,
               int(vocab_size))
        info = self._prepare(seq_lens, weight_indices, lora_ranks, scalings, is_decode,
                             use_cuda_graph, chunk_size_override, emb)
        return info, out

    def _prepare(self, seq_lens, weight_indices, lora_ranks, scalings, is_decode,
                 use_cuda_graph, chunk_size_override, emb):
        L = self.max_loras_per_batch
        lens, slots, ranks, scal, s = batch_arrays(seq_lens, weight_indices, lora_ranks,
                                                   scalings, L)
        if emb is not None and emb[0] != s:
            raise ValueError(f"{emb[0]} ids, the batch has {s} tokens")
        bs = len(slots)
        if use_cuda_graph:
            if self._graph_cap is None:
                raise RuntimeError("call init_cuda_graph_batch_info first")
            max_bs, max_tokens, seg_cap = self._graph_cap
            if bs > max_bs or s > max_tokens:
                raise ValueError("batch exceeds the graph capacity")
            s_cap, req_cap = max_tokens, max_bs
        else:
            min_chunk = chunk_size_override if chunk_size_override > 0 else MIN_CHUNK_SIZE
            seg_cap = self._seg_caps.get((s, min_chunk))
            if seg_cap is None:
                seg_cap = B.lora_plan_max_segments(s, L, min_chunk)
                if len(self._seg_caps) < 4096:
                    self._seg_caps[(s, min_chunk)] = seg_cap
            s_cap, req_cap = s, bs
        key = (s_cap, seg_cap, req_cap)
        total, regions = self._layout(s_cap, seg_cap, req_cap)
        stg = self._staging
        ring = stg.take(total)
        if use_cuda_graph:
            dev = self._graph_dev
            dev_addr, dev_bytes = dev.data_ptr(), 4 * dev.numel()
        else:
            dev, dev_addr, dev_bytes = stg.dev[ring], stg.dev_addr[ring], stg.dev_bytes[ring]
        idx = self._dev_index if self._dev_index is not None else torch.cuda.current_device()
        stream = torch._C._cuda_getCurrentRawStream(idx)
        flag, flag_value = stg.signal(ring)
        if emb is None:
            check(calls().lora_plan_upload(
                lens, slots, bs, ranks, scal, L, 1 if is_decode else 0, self.max_chunk_size,
                int(chunk_size_override), s_cap, seg_cap, req_cap, stg.host_addr[ring],
                dev_addr, dev_bytes, self._info_addr, flag, flag_value, stream))
        else:
            check(calls().lora_plan_upload_embedding(
                lens, slots, bs, ranks, scal, L, 1 if is_decode else 0, self.max_chunk_size,
                int(chunk_size_override), s_cap, seg_cap, req_cap, stg.host_addr[ring],
                dev_addr, dev_bytes, self._info_addr, flag, flag_value, *emb[1:], stream))
        stg.done(ring)
        n_seg, chunk, longest, _, n_work, longest_work = self._info_np.tolist()
        if use_cuda_graph:
            # fixed views and launch shape: capacity segments over capacity tokens
            batch = self.cuda_graph_batch_info
            batch.bs, batch.max_len, batch.planned_segments = bs, chunk, n_seg
            batch.planned_tokens = s
            self.batch_info = batch
            return batch
        # eager: the views of a layout are built once, for every slot of the
        # ring at the same time, and reused
        batch = stg.infos[ring].get(key)
        if batch is None:
            for i in range(stg.n):
                d = stg.dev[i]
                v = {name: d[o:o + n] for name, (o, n) in zip(_NAMES, regions)}
                stg.infos[i][key] = LoRABatchInfo(
                    bs=bs, num_tokens=s, num_segments=0, max_len=chunk,
                    seg_indptr=v["seg_indptr"], weight_indices=v["seg_slots"],
                    permutation=v["permutation"], lora_ranks=v["ranks"],
                    scalings=v["scalings"].view(torch.float32),
                    req_seg_indptr=v["req_seg_indptr"], req_weight_indices=v["req_slots"],
                    use_cuda_graph=False, work_indptr=v["work_indptr"],
                    work_slots=v["work_slots"])
            batch = stg.infos[ring][key]
        batch.bs = bs
        batch.num_segments, batch.max_len, batch.max_seg_len = n_seg, chunk, longest
        batch.num_work_segments, batch.max_work_len = n_work, longest_work
        batch.planned_segments = n_seg
        batch.planned_tokens = s
        self.batch_info = batch
        return batch

    # ------------------------------------------------------------ lm_head
    def prepare_lm_head_batch(self, pruned_lens, weight_indices, lora_ranks, scalings,
                              chunk_size_override=0):
        """Plan and upload the pruned lm_head pass (``_prepare_lm_head_batch_info``):
        ``pruned_lens[r]`` tokens of request r reach the lm_head, in original
        order (identity permutation); segments are runs of consecutive
        same-slot requests cut into chunks.  The result is also kept as
        ``lm_head_batch_info``; pass it as ``pruned_batch_info`` to
        run_lora_a_sgemm / run_lora_b_sgemm."""
        batch = self._lm_head_plan(pruned_lens, weight_indices, lora_ranks, scalings,
                                   chunk_size_override)
        self.lm_head_batch_info = batch
        return batch

    def prepare_lm_head_pass_batches(self, passes, lora_ranks, scalings):
        """Per-pass lm_head plans for logprob chunking: one plan per
        (weight_indices, pruned_lens) pass, each over that pass's requests
        (the page plans each pass the same way as the whole batch)."""
        out = [self._lm_head_plan(lens, wi, lora_ranks, scalings, 0) for wi, lens in passes]
        self.lm_head_pass_batch_infos = out
        return out

    def _lm_head_plan(self, pruned_lens, weight_indices, lora_ranks, scalings, override):
        L = self.max_loras_per_batch
        if pruned_lens is None:
            raise ValueError("pruned_lens is required")
        lens, slots, ranks, scal, s = batch_arrays(pruned_lens, weight_indices, lora_ranks,
                                                   scalings, L)
        bs = len(slots)
        min_chunk = override if override > 0 else MIN_CHUNK_SIZE
        # runs of consecutive requests are not bounded by the slot count
        seg_cap = B.lora_plan_max_segments(s, max(bs, 1), min_chunk)
        total, regions = self._layout(s, seg_cap, bs)
        stg = self._staging
        ring = stg.take(total)
        dev = stg.dev[ring]
        idx = self.device.index if self.device.index is not None else torch.cuda.current_device()
        stream = torch._C._cuda_getCurrentRawStream(idx)
        info = self._info_arr
        flag, flag_value = stg.signal(ring)
        check(calls().lora_plan_lm_head_upload(
            lens.ctypes.data, slots.ctypes.data, bs, ranks.ctypes.data, scal.ctypes.data, L,
            self.max_chunk_size, int(override), s, seg_cap, bs, stg.host[ring].data_ptr(),
            dev.data_ptr(), 4 * dev.numel(), self._info_addr, flag, flag_value, stream))
        stg.done(ring)
        n_seg, chunk, longest, n_work, longest_work = info[0], info[1], info[2], info[4], info[5]
        v = {name: dev[o:o + n] for name, (o, n) in zip(_NAMES, regions)}
        # a fresh LoRABatchInfo (not one of the eager step's cached views)
        return LoRABatchInfo(
            bs=bs, num_tokens=s, num_segments=n_seg, max_len=chunk,
            seg_indptr=v["seg_indptr"], weight_indices=v["seg_slots"],
            permutation=v["permutation"], lora_ranks=v["ranks"],
            scalings=v["scalings"].view(torch.float32), req_seg_indptr=v["req_seg_indptr"],
            req_weight_indices=v["req_slots"], use_cuda_graph=False, max_seg_len=longest,
            work_indptr=v["work_indptr"], work_slots=v["work_slots"], num_work_segments=n_work,
            max_work_len=longest_work, work_perm=v["work_perm"])

    def init_cuda_graph_batch_info(self, max_bs_in_cuda_graph, num_tokens_per_bs):
        """Preallocate fixed-capacity device plan arrays for graph capture.

        Capacity: the page's ceil(tokens_per_bs / 16) segments per request,
        or the tighter bound ceil(tokens / 16) + max_loras when smaller (no
        plan can exceed either).  Unused segments are padded to zero length
        with slot 0, and kernels are launched over the full capacity so the
        launch shape never changes between replays.
        """
        max_tokens = max_bs_in_cuda_graph * num_tokens_per_bs
        cap = (num_tokens_per_bs + MIN_CHUNK_SIZE - 1) // MIN_CHUNK_SIZE * max_bs_in_cuda_graph
        cap = min(cap, B.lora_plan_max_segments(max_tokens, self.max_loras_per_batch,
                                                MIN_CHUNK_SIZE))
        self._graph_cap = (max_bs_in_cuda_graph, max_tokens, cap)
        total, regions = self._layout(max_tokens, cap, max_bs_in_cuda_graph)
        dev = torch.zeros(total, dtype=torch.int32, device=self.device)
        self._graph_dev = dev
        v = {name: dev[o:o + n] for name, (o, n) in zip(_NAMES, regions)}
        # Kernels see the capacity: num_segments = cap (padding segments are
        # empty) and num_tokens = max_tokens (activations are allocated for
        # the capacity).
        # typical segment length (tokens per adapter slot); longer segments
        # are still covered, by the same workgroups looping
        cap_chunk = max(MIN_CHUNK_SIZE, min(self.max_chunk_size, 128))
        per_slot = -(-max_tokens // max(self.max_loras_per_batch, 1))
        hint = max(MIN_CHUNK_SIZE, min(cap_chunk, -(-per_slot // 16) * 16))
        self.cuda_graph_batch_info = LoRABatchInfo(
            bs=max_bs_in_cuda_graph, num_tokens=max_tokens, num_segments=cap,
            max_len=hint, seg_indptr=v["seg_indptr"], weight_indices=v["seg_slots"],
            permutation=v["permutation"], lora_ranks=v["ranks"],
            scalings=v["scalings"].view(torch.float32), req_seg_indptr=v["req_seg_indptr"],
            req_weight_indices=v["req_slots"], use_cuda_graph=True, max_seg_len=hint,
            work_indptr=v["work_indptr"], work_slots=v["work_slots"], num_work_segments=cap,
            max_work_len=hint)
        return self.cuda_graph_batch_info

    def prepare_lora_batch_device(self, seq_lens, weight_indices, lora_ranks, scalings,
                                  is_decode=False, chunk_size_override=0):
        """Plan into the graph buffer on the GPU (lora_plan_device) from
        device tensors: no host round trip, so a graph may capture this call
        together with the kernels; update the tensors' contents between
        replays.  Needs init_cuda_graph_batch_info; the batch size is
        weight_indices.numel() (at most the graph's).  The plan's counts and
        status are left in ``cuda_graph_plan_info`` (int32 [8], device)."""
        if self._graph_cap is None:
            raise RuntimeError("call init_cuda_graph_batch_info first")
        max_bs, max_tokens, seg_cap = self._graph_cap
        if weight_indices.numel() > max_bs:
            raise ValueError("batch exceeds the graph capacity")
        if self._graph_info_dev is None:
            self._graph_info_dev = torch.zeros(8, dtype=torch.int32, device=self.device)
        B.lora_plan_device(seq_lens, weight_indices, lora_ranks, scalings,
                           self.max_loras_per_batch, is_decode, self.max_chunk_size,
                           chunk_size_override, max_tokens, seg_cap, max_bs, self._graph_dev,
                           self._graph_info_dev)
        self.cuda_graph_plan_info = self._graph_info_dev
        self.batch_info = self.cuda_graph_batch_info
        return self.cuda_graph_batch_info

    def prepare_moe_lora_batch(self, topk_ids, num_experts, batch_info=None):
        """The plan of a MoE LoRA add (PR #24007 report page: the MoE layer
        reads each token's adapter from the per-request fields
        req_seg_indptr / req_weight_indices and combines it with the
        router's experts into "virtual experts").  On the GPU, with no host
        round trip, in one launch (lora_moe_plan): every top-k copy t*k + j of
        a token gets its virtual expert a(t) * E + topk_ids[t, j], and the
        copies are planned like a decode batch of one-token requests (the
        copies' virtual experts are the plan's req_weight_indices).
        topk_ids: int32 (num_tokens, k) device tensor of the batch's tokens
        (batch_info: the current plan unless given).  The result's arrays
        are padded to a fixed capacity, so a graph may capture this call
        with the kernels; the plan's counts and status are left in
        ``moe_plan_info`` (int32 [8], device).  Capacity of the device
        planner: num_tokens * k <= 4096 copies, L * E < 1024."""
        info = self._info(batch_info)
        if info.req_seg_indptr is None or info.req_weight_indices is None:
            raise ValueError("the batch plan has no per-request routing fields")
        if topk_ids.dim() != 2 or topk_ids.dtype != torch.int32 or not topk_ids.is_cuda:
            raise TypeError("topk_ids must be an int32 (num_tokens, k) device tensor")
        s, k = topk_ids.shape
        if s != info.num_tokens:
            raise ValueError(f"topk_ids has {s} rows, the batch has {info.num_tokens} tokens")
        L, E = self.max_loras_per_batch, int(num_experts)
        nv = L * E + 1
        copies = s * k
        seg_cap = B.lora_plan_max_segments(copies, nv, MIN_CHUNK_SIZE)
        key = (copies, E)
        bufs = self._moe.get(key)
        if bufs is None:
            offs = (ctypes.c_int64 * len(_NAMES))()
            total = int(lib().lora_plan_layout(copies, seg_cap, copies, nv, offs))
            sizes = (copies, seg_cap + 1, seg_cap, copies + 1, copies, nv, nv, seg_cap + 1,
                     seg_cap, copies)
            plan = torch.zeros(max(total, 1), dtype=torch.int32, device=self.device)
            v = {name: plan[int(o):int(o) + n] for name, o, n in zip(_NAMES, offs, sizes)}
            bufs = {"plan": plan, "v": v,
                    "info": torch.zeros(8, dtype=torch.int32, device=self.device)}
            self._moe[key] = bufs
        B.lora_moe_plan(info.req_seg_indptr, info.req_weight_indices, info.bs, topk_ids, E,
                        info.lora_ranks, info.scalings, L, self.max_chunk_size, seg_cap,
                        bufs["plan"], bufs["info"])
        v = bufs["v"]
        # typical segment length: copies per virtual expert, in whole 16-token
        # tiles between 16 and 128 (longer segments are still covered)
        per_expert = -(-copies // max(L * E, 1))
        hint = max(MIN_CHUNK_SIZE, min(128, -(-per_expert // 16) * 16))
        self.moe_plan_info = bufs["info"]
        self.moe_batch_info = LoRABatchInfo(
            bs=copies, num_tokens=copies, num_segments=seg_cap, max_len=hint,
            seg_indptr=v["seg_indptr"], weight_indices=v["seg_slots"],
            permutation=v["permutation"], lora_ranks=v["ranks"],
            scalings=v["scalings"].view(torch.float32), req_seg_indptr=v["req_seg_indptr"],
            req_weight_indices=v["req_slots"], use_cuda_graph=True, max_seg_len=hint,
            work_indptr=v["work_indptr"],
            work_slots=v["work_slots"], num_work_segments=seg_cap, max_work_len=hint)
        return self.moe_batch_info

    def run_moe_lora_add(self, x, moe_lora_a, moe_lora_b, intermediate, top_k, moe_info=None,
                         workspace=None):
        """Add the LoRA deltas of a MoE layer into the fused-MoE intermediate
        (num_tokens * top_k rows, row t*top_k + j for token t's j-th expert):
        moe_lora_a (L, E, R, K), moe_lora_b (L, E, N, R)."""
        info = moe_info if moe_info is not None else self.moe_batch_info
        if info is None:
            raise RuntimeError("prepare_moe_lora_batch has not been called")
        return B.lora_moe_add(x, moe_lora_a, moe_lora_b, info, top_k, intermediate, workspace)

    # -------------------------------------------------------------- kernels
    def _info(self, pruned_batch_info=None):
        info = pruned_batch_info if pruned_batch_info is not None else self.batch_info
        if info is None:
            raise RuntimeError("prepare_lora_batch has not been called")
        return info

    def run_lora_a_sgemm(self, x, weights, pruned_batch_info=None, stack_num=1, **_):
        return B.lora_shrink(x, weights, self._info(pruned_batch_info), num_slices=stack_num)

    def run_lora_b_sgemm(self, x, weights, output_offset=None, base_output=None,
                         pruned_batch_info=None, **_):
        out_dim = weights.shape[-2]
        offs = [0, out_dim] if output_offset is None else output_offset
        return B.lora_expand(x, weights, self._info(pruned_batch_info), offs, out_dim,
                             base_output)

    def run_qkv_lora(self, x, qkv_lora_a, qkv_lora_b, output_offset, max_qkv_out_dim,
                     base_output=None, n_slices=3, **_):
        if not isinstance(qkv_lora_b, torch.Tensor):
            raise TypeError("qkv_lora_b must be one stacked tensor")
        offs = np.asarray(output_offset.cpu() if isinstance(output_offset, torch.Tensor)
                          else output_offset, dtype=np.int32)
        if len(offs) != n_slices + 1:
            raise ValueError(f"output_offset needs {n_slices + 1} entries")
        return B.lora_qkv(x, qkv_lora_a, qkv_lora_b, self._info(), offs, max_qkv_out_dim,
                          base_output)

    def run_gate_up_lora(self, x, gate_up_lora_a, gate_up_lora_b, output_offset=None,
                         base_output=None, **_):
        if not isinstance(gate_up_lora_b, torch.Tensor):
            raise TypeError("gate_up_lora_b must be one stacked tensor")
        out_dim = gate_up_lora_b.shape[-2] // 2
        offs = [0, out_dim, 2 * out_dim] if output_offset is None else output_offset
        return B.lora_qkv(x, gate_up_lora_a, gate_up_lora_b, self._info(), offs, out_dim,
                          base_output)

    def run_lora_a_embedding(self, input_ids, weights, vocab_size, extra_embeddings=None, **_):
        if extra_embeddings is not None:
            raise NotImplementedError(
                "extra (added-vocabulary) embeddings are not supported by the chunked backend")
        return B.lora_a_embedding(input_ids, weights, self._info(), vocab_size)

    def run_extra_token_embedding(self, *args, **kwargs):
        raise NotImplementedError("extra token embeddings are not supported")


__all__ = ["ChunkedSgmvLoRA", "LoRABatchInfo"]
