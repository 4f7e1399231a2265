"""ChunkedSgmvLoRA: the chunked SGMV LoRA backend API over the C ABI.

Method names and arguments follow the ``ChunkedSgmvLoRABackend`` /
``BaseLoRABackend`` pages (prepare_lora_batch, run_lora_a_sgemm,
run_lora_b_sgemm, run_qkv_lora, run_gate_up_lora, run_lora_a_embedding,
init_cuda_graph_batch_info).  Every step of the work runs in libsgg_lora:
the plan in its host planner, the rest in its HIP kernels.

Upload: the page copies six small host arrays to the device one by one.
Here the planner writes every plan array into one pinned staging buffer and a
single non-blocking host-to-device copy moves them; the device arrays are
views of one device buffer.  Staging buffers rotate through a small ring and
are reused only after the copy that last read them has completed, so
planning the next batch never waits for the GPU.
"""

import numpy as np
import torch

from . import binding as B
from .binding import LoRABatchInfo

MIN_CHUNK_SIZE = 16


def _align(n, m=64):
    return (n + m - 1) // m * m


class _Staging:
    """Ring of pinned int32 buffers, each guarded by the event of its last copy."""

    def __init__(self, slots=3):
        self.bufs = [None] * slots
        self.events = [None] * slots
        self.i = 0

    def take(self, n):
        i = self.i
        self.i = (i + 1) % len(self.bufs)
        if self.events[i] is not None:
            self.events[i].synchronize()
        if self.bufs[i] is None or self.bufs[i].numel() < n:
            self.bufs[i] = torch.empty(max(n, 1024), dtype=torch.int32, pin_memory=True)
        return i, self.bufs[i]

    def done(self, i, stream):
        ev = torch.cuda.Event()
        ev.record(stream)
        self.events[i] = ev


class ChunkedSgmvLoRA:
    """Chunked segmented-gather LoRA backend for one device."""

    name = "csgmv"

    def __init__(self, max_loras_per_batch, max_chunk_size=128, device="cuda"):
        self.max_loras_per_batch = int(max_loras_per_batch)
        self.max_chunk_size = int(max_chunk_size)
        self.device = torch.device(device)
        self.batch_info = None
        self.cuda_graph_batch_info = None
        self._graph_dev = None
        self._graph_cap = None
        self._staging = _Staging()

    # ---------------------------------------------------------------- plan
    def _layout(self, s, cap, bs):
        L = self.max_loras_per_batch
        off = {}
        pos = 0
        for name, n in (("permutation", s), ("seg_indptr", cap + 1), ("seg_slots", cap),
                        ("req_seg_indptr", bs + 1), ("req_slots", bs), ("ranks", L),
                        ("scalings", L)):
            off[name] = (pos, n)
            pos += _align(n)
        return off, pos

    def prepare_lora_batch(self, seq_lens, weight_indices, lora_ranks, scalings,
                           is_decode=False, use_cuda_graph=False, chunk_size_override=0):
        """Plan the batch on the host and upload it with one async copy.

        seq_lens: tokens per request (None in decode mode: one each);
        weight_indices: slot per request; lora_ranks / scalings: per slot
        (``max_loras_per_batch`` entries, rank 0 = no adapter).
        """
        L = self.max_loras_per_batch
        if len(lora_ranks) != L or len(scalings) != L:
            raise ValueError(f"lora_ranks and scalings need {L} entries")
        bs = len(weight_indices)
        s = bs if seq_lens is None else int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
        if use_cuda_graph:
            if self._graph_cap is None:
                raise RuntimeError("call init_cuda_graph_batch_info first")
            max_bs, max_tokens, cap = self._graph_cap
            if bs > max_bs or s > max_tokens:
                raise ValueError("batch exceeds the graph capacity")
            s_alloc, bs_alloc = max_tokens, max_bs
        else:
            min_chunk = chunk_size_override if chunk_size_override > 0 else MIN_CHUNK_SIZE
            cap = B.lora_plan_max_segments(s, L, min_chunk)
            s_alloc, bs_alloc = s, bs
        off, total = self._layout(s_alloc, cap, bs_alloc)
        slot, buf = self._staging.take(total)

        def view(name, n=None):
            o, size = off[name]
            return buf[o:o + (size if n is None else n)]

        plan = B.lora_plan_segments(
            seq_lens, weight_indices, L, is_decode, self.max_chunk_size, chunk_size_override,
            seg_capacity=cap,
            out={"permutation": view("permutation", max(s, 1)),
                 "seg_indptr": view("seg_indptr"), "seg_slots": view("seg_slots"),
                 "req_seg_indptr": view("req_seg_indptr", bs + 1)})
        view("req_slots", bs).copy_(torch.as_tensor(np.asarray(weight_indices, np.int32)))
        view("ranks").copy_(torch.as_tensor(np.asarray(lora_ranks, np.int32)))
        view("scalings").copy_(torch.as_tensor(np.asarray(scalings, np.float32)).view(torch.int32))

        stream = torch.cuda.current_stream(self.device)
        if use_cuda_graph:
            dev = self._graph_dev
        else:
            dev = torch.empty(total, dtype=torch.int32, device=self.device)
        dev[:total].copy_(buf[:total], non_blocking=True)
        self._staging.done(slot, stream)

        def dview(name, n=None):
            o, size = off[name]
            return dev[o:o + (size if n is None else n)]

        n_seg = plan["num_segments"]
        indptr = view("seg_indptr")[:n_seg + 1].numpy()
        longest = int((indptr[1:] - indptr[:-1]).max()) if n_seg > 0 else 0
        info = LoRABatchInfo(
            bs=bs, num_tokens=s,
            num_segments=cap if use_cuda_graph else n_seg,
            max_len=plan["chunk_size"],
            seg_indptr=dview("seg_indptr"), weight_indices=dview("seg_slots"),
            permutation=dview("permutation", s), lora_ranks=dview("ranks"),
            scalings=dview("scalings").view(torch.float32),
            req_seg_indptr=dview("req_seg_indptr", bs + 1),
            req_weight_indices=dview("req_slots", bs), use_cuda_graph=use_cuda_graph,
            max_seg_len=0 if use_cuda_graph else longest)
        info.planned_segments = n_seg
        self.batch_info = info
        return info

    def init_cuda_graph_batch_info(self, max_bs_in_cuda_graph, num_tokens_per_bs):
        """Preallocate fixed-capacity device plan arrays for graph capture.

        Capacity follows the page: ceil(tokens_per_bs / 16) segments per
        request; unused segments are padded to zero length with slot 0, and
        kernels are always launched over the full capacity so the launch
        shape never changes between replays.
        """
        max_tokens = max_bs_in_cuda_graph * num_tokens_per_bs
        cap = (num_tokens_per_bs + MIN_CHUNK_SIZE - 1) // MIN_CHUNK_SIZE * max_bs_in_cuda_graph
        cap = max(cap, B.lora_plan_max_segments(max_tokens, self.max_loras_per_batch,
                                                MIN_CHUNK_SIZE))
        self._graph_cap = (max_bs_in_cuda_graph, max_tokens, cap)
        _, total = self._layout(max_tokens, cap, max_bs_in_cuda_graph)
        self._graph_dev = torch.zeros(total, dtype=torch.int32, device=self.device)

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
