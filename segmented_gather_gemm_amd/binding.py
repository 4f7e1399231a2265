"""Thin Python binding over the C ABI: argument marshalling only.

Each function has the name of the C entry point it calls and does no
arithmetic of its own.  Tensors must be bf16 (int32 / int64 / float32 for
plan arrays, ids and scalings) on a ROCm device; the call is enqueued on
torch's current stream of that device.
"""

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from ._lib import calls, check, lib

_P32 = ctypes.POINTER(ctypes.c_int32)
_P64 = ctypes.POINTER(ctypes.c_int64)


@dataclass
class LoRABatchInfo:
    """Device-resident plan of one batch (the pages' LoRABatchInfo fields).

    ``weight_indices`` is the per-segment slot array, ``max_len`` the chunk
    size.  Segment arrays may be longer than ``num_segments`` (padding).
    """
    bs: int
    num_tokens: int
    num_segments: int
    max_len: int
    seg_indptr: torch.Tensor
    weight_indices: torch.Tensor
    permutation: torch.Tensor
    lora_ranks: torch.Tensor
    scalings: torch.Tensor
    req_seg_indptr: Optional[torch.Tensor] = None
    req_weight_indices: Optional[torch.Tensor] = None
    use_cuda_graph: bool = False
    max_seg_len: int = 0          # longest planned segment (0: unknown, use max_len)
    # Work decomposition (optional): segments with consecutive segments of
    # one slot merged, over `work_perm` (None: the plan's permutation; an
    # lm_head plan's tokens sorted by slot); kernels run over it when present,
    # with the same results (lora_plan_upload, lora_plan_lm_head_upload).
    work_indptr: Optional[torch.Tensor] = None
    work_slots: Optional[torch.Tensor] = None
    num_work_segments: int = 0
    max_work_len: int = 0
    work_perm: Optional[torch.Tensor] = None

    @property
    def tile_hint(self):
        """Upper bound on segment length handed to the kernels for tiling."""
        return self.max_seg_len if self.max_seg_len > 0 else self.max_len

    def kernel_segments(self):
        """(indptr, slots, count, tile hint, permutation) of the decomposition
        the kernels run over."""
        if self.work_indptr is not None:
            hint = self.max_work_len if self.max_work_len > 0 else self.tile_hint
            perm = self.permutation if self.work_perm is None else self.work_perm
            return self.work_indptr, self.work_slots, self.num_work_segments, hint, perm
        return (self.seg_indptr, self.weight_indices, self.num_segments, self.tile_hint,
                self.permutation)


def _vp(t):
    """Device address of a tensor (0 for None), passed as an integer."""
    return t.data_ptr() if t is not None else 0


def _stream(t):
    """Raw handle of torch's current stream on the device of tensor `t` (the
    launch stream)."""
    return torch._C._cuda_getCurrentRawStream(t.get_device())


def _host_i32(values):
    arr = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return arr, arr.ctypes.data_as(_P32)


def _cpu_i32_ptr(t):
    if t is None:
        return ctypes.cast(0, _P32)
    if t.dtype != torch.int32 or t.device.type != "cpu" or not t.is_contiguous():
        raise ValueError("plan output arrays must be contiguous int32 CPU tensors")
    return ctypes.cast(t.data_ptr(), _P32)


def _need_bf16(name, t, dims):
    """A bf16 device tensor of `dims` dimensions with unit stride in its last
    one; returns its strides (one query: each stride(i) call costs as much)."""
    st = t.stride()
    if t.dtype is not torch.bfloat16 or not t.is_cuda or len(st) != dims or st[-1] != 1:
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a ROCm device")
        if t.dim() != dims:
            raise ValueError(f"{name} must have {dims} dimensions, got shape {tuple(t.shape)}")
        raise ValueError(f"{name} must have unit stride in its last dimension")
    return st


def _need_bf16_dense(name, t, dims):
    """A dense bf16 device tensor of `dims` dimensions (weights)."""
    if t.dtype is not torch.bfloat16 or not t.is_cuda or t.dim() != dims or not t.is_contiguous():
        _need_bf16(name, t, dims)
        _need_dense(name, t)


def _need_rows_cols(name, t, rows, cols):
    """`t` holds at least `rows` x `cols` elements (the kernels write them)."""
    shape = t.shape
    if shape[0] != rows or shape[1] < cols:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, needs ({rows}, >= {cols})")


def _need_dense(name, t):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def lora_plan_max_segments(num_tokens, max_loras, min_chunk=16):
    return calls().lora_plan_max_segments(int(num_tokens), int(max_loras), int(min_chunk))


def lora_plan_segments(seq_lens, req_slots, max_loras, is_decode, max_chunk_size,
                       chunk_size_override=0, seg_capacity=None, out=None):
    """Plan a batch on the host.

    ``out`` may hold preallocated contiguous int32 CPU tensors ``permutation``,
    ``seg_indptr``, ``seg_slots``, ``req_seg_indptr`` (e.g. views of one
    pinned staging buffer); otherwise NumPy arrays are allocated.  Returns a
    dict with those arrays and ``num_segments``, ``chunk_size``,
    ``num_tokens``.
    """
    slots, p_slots = _host_i32(req_slots)
    bs = len(slots)
    if seq_lens is None:
        lens, p_lens = None, ctypes.cast(0, _P32)
        s_hint = bs
    else:
        lens, p_lens = _host_i32(seq_lens)
        if len(lens) != bs:
            raise ValueError("seq_lens and req_slots differ in length")
        s_hint = int(lens.astype(np.int64).sum())
    min_chunk = chunk_size_override if chunk_size_override > 0 else 16
    cap = (lora_plan_max_segments(s_hint, max_loras, min_chunk)
           if seg_capacity is None else int(seg_capacity))
    if out is None:
        out = {"permutation": np.zeros(max(s_hint, 1), np.int32),
               "seg_indptr": np.zeros(cap + 1, np.int32),
               "seg_slots": np.zeros(max(cap, 1), np.int32),
               "req_seg_indptr": np.zeros(bs + 1, np.int32)}

    def ptr(a):
        if isinstance(a, np.ndarray):
            return a.ctypes.data_as(_P32)
        return _cpu_i32_ptr(a)

    n_seg, chunk, n_tok = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    perm = out["permutation"]
    check(lib().lora_plan_segments(
        p_lens, p_slots, bs, int(max_loras), 1 if is_decode else 0, int(max_chunk_size),
        int(chunk_size_override), ptr(perm), int(perm.shape[0]) if s_hint else 0,
        ptr(out["seg_indptr"]), ptr(out["seg_slots"]), cap, ptr(out["req_seg_indptr"]),
        ctypes.byref(n_seg), ctypes.byref(chunk), ctypes.byref(n_tok)))
    res = dict(out)
    res.update(num_segments=n_seg.value, chunk_size=chunk.value, num_tokens=n_tok.value,
               capacity=cap)
    return res


def lora_plan_lm_head(pruned_lens, req_slots, max_loras, max_chunk_size, chunk_size_override=0,
                      seg_capacity=None):
    """Plan a pruned lm_head pass on the host (identity permutation).

    Returns a dict with ``permutation``, ``seg_indptr``, ``seg_slots`` (NumPy
    arrays), ``num_segments``, ``chunk_size``, ``num_tokens``, ``capacity``.
    """
    slots, p_slots = _host_i32(req_slots)
    lens, p_lens = _host_i32(pruned_lens)
    if len(lens) != len(slots):
        raise ValueError("pruned_lens and req_slots differ in length")
    s = int(lens.astype(np.int64).sum())
    min_chunk = chunk_size_override if chunk_size_override > 0 else 16
    cap = (lora_plan_max_segments(s, max(len(slots), 1), min_chunk)
           if seg_capacity is None else int(seg_capacity))
    perm = np.zeros(max(s, 1), np.int32)
    ind = np.zeros(cap + 1, np.int32)
    sl = np.zeros(max(cap, 1), np.int32)
    n_seg, chunk, n_tok = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    check(lib().lora_plan_lm_head(
        p_lens, p_slots, len(slots), int(max_loras), int(max_chunk_size),
        int(chunk_size_override), perm.ctypes.data_as(_P32), s, ind.ctypes.data_as(_P32),
        sl.ctypes.data_as(_P32), cap, ctypes.byref(n_seg), ctypes.byref(chunk),
        ctypes.byref(n_tok)))
    return {"permutation": perm[:s], "seg_indptr": ind, "seg_slots": sl,
            "num_segments": n_seg.value, "chunk_size": chunk.value, "num_tokens": n_tok.value,
            "capacity": cap}


def lora_plan_device(seq_lens, req_slots, lora_ranks, scalings, max_loras, is_decode,
                     max_chunk_size, chunk_size_override, token_capacity, seg_capacity,
                     req_capacity, device_plan, device_info):
    """Plan a batch on the GPU into `device_plan` (int32 device tensor in the
    lora_plan_layout layout) from device tensors: seq_lens (int32, ignored in
    decode mode), req_slots (int32), lora_ranks (int32) and scalings
    (float32).  The counts and a status go to device_info (int32 [8]) on the
    device; nothing is copied to the host."""
    def dev_i32(name, t, n):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.numel() < n:
            raise ValueError(f"{name} must be a contiguous int32 device tensor of >= {n} entries")
    bs = req_slots.numel()
    dev_i32("req_slots", req_slots, bs)
    if not is_decode:
        dev_i32("seq_lens", seq_lens, bs)
    dev_i32("lora_ranks", lora_ranks, max_loras)
    dev_i32("device_plan", device_plan, 1)
    dev_i32("device_info", device_info, 8)
    if scalings.dtype != torch.float32 or not scalings.is_cuda or not scalings.is_contiguous() \
            or scalings.numel() < max_loras:
        raise ValueError("scalings must be a contiguous float32 device tensor")
    check(calls().lora_plan_device(
        None if is_decode else seq_lens.data_ptr(), req_slots.data_ptr(), bs,
        lora_ranks.data_ptr(), scalings.data_ptr(), int(max_loras), 1 if is_decode else 0,
        int(max_chunk_size), int(chunk_size_override), int(token_capacity), int(seg_capacity),
        int(req_capacity), device_plan.data_ptr(), 4 * device_plan.numel(),
        device_info.data_ptr(), _stream(device_plan)))


def lora_set_option(name, value):
    """Process-wide setting of the device calls ("fused_stacked": 1/0,
    "spin_limit": polls); returns the previous value."""
    old = lib().lora_set_option(name.encode(), int(value))
    if old < 0:
        raise ValueError(f"unknown option {name!r}")
    return old


# ----------------------------------------------------------------- workspace

_workspaces = {}
_outgrown = []


def default_workspace(device, nbytes):
    """A zero-initialised, grow-only scratch buffer per device.

    A workspace that a larger call outgrows is kept alive, never freed: a
    graph captured with it keeps its address and would otherwise write its
    split-K counters, partials and h into memory another tensor may own.
    Growth doubles, so all of them together take at most twice the largest.
    Calls that use the same workspace must not overlap: use it from one
    stream, or pass a separate workspace per stream.
    """
    device = torch.device(device)
    key = (device.type, device.index if device.index is not None else torch.cuda.current_device())
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(int(nbytes), 1 << 20)
        if ws is not None:
            size = max(size, 2 * ws.numel())
            _outgrown.append(ws)
        ws = torch.zeros(size, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


_offset_cache = {}


def _offsets(slice_offsets):
    """Host int32 copy of the slice offsets and its address (cached for lists and tuples)."""
    key = tuple(slice_offsets) if isinstance(slice_offsets, (list, tuple)) else None
    if key is not None:
        hit = _offset_cache.get(key)
        if hit is not None:
            return hit
    if isinstance(slice_offsets, torch.Tensor):
        slice_offsets = slice_offsets.detach().to("cpu")  # host copy (synchronises if on device)
    arr = np.ascontiguousarray(np.asarray(slice_offsets, dtype=np.int32))
    if arr.ndim != 1 or len(arr) < 2:
        raise ValueError("slice_offsets needs at least two entries")
    hit = (arr, arr.ctypes.data)
    if key is not None and len(_offset_cache) < 256:
        _offset_cache[key] = hit
    return hit


# ---------------------------------------------------------------- device calls

def lora_shrink(x, weights, batch_info: LoRABatchInfo, num_slices=1, out=None, workspace=None):
    """LoRA-A: x (s, K), weights (L, c*R, K) -> h (s, c*R), original token order."""
    xst = _need_bf16("x", x, 2)
    _need_bf16_dense("weights", weights, 3)
    s, K = x.shape
    L, CR, K2 = weights.shape
    if K2 != K:
        raise ValueError(f"weights in_dim {K2} != x in_dim {K}")
    if CR % num_slices:
        raise ValueError(f"weights rows {CR} not a multiple of num_slices {num_slices}")
    if s != batch_info.num_tokens:
        raise ValueError(f"x has {s} rows, the plan has {batch_info.num_tokens} tokens")
    R = CR // num_slices
    if out is None:
        out = torch.empty((s, CR), dtype=torch.bfloat16, device=x.device)
    ost = _need_bf16("out", out, 2)
    _need_rows_cols("out", out, s, CR)
    ind, sl, nseg, hint, perm = batch_info.kernel_segments()
    ws = workspace
    if ws is None:   # the library checks the size of a caller's workspace itself
        need = calls().lora_shrink_workspace_bytes(s, K, num_slices, R, nseg, hint)
        ws = default_workspace(x.device, need) if need else None
    check(calls().lora_shrink(
        _vp(x), xst[0], _vp(weights), _vp(out), ost[0], s, K, L, num_slices, R,
        _vp(ind), _vp(sl), nseg, _vp(perm), _vp(batch_info.lora_ranks), hint,
        _vp(ws), ws.numel() if ws is not None else 0, _stream(x)))
    return out


def lora_expand(h, weights, batch_info: LoRABatchInfo, slice_offsets, max_slice_size,
                base_output=None):
    """LoRA-B: base_output[:, o_k:o_{k+1}] += scaling * h-slice k @ B-slice k^T, in place.

    ``base_output=None`` gives a zero-filled output (the update alone).
    """
    hst = _need_bf16("h", h, 2)
    _need_bf16_dense("weights", weights, 3)
    offs, p_offs = _offsets(slice_offsets)
    c = len(offs) - 1
    s = h.shape[0]
    L, N, R = weights.shape
    if s != batch_info.num_tokens:
        raise ValueError(f"h has {s} rows, the plan has {batch_info.num_tokens} tokens")
    _need_rows_cols("h", h, s, c * R)
    if base_output is None:
        base_output = torch.zeros((s, int(offs[-1])), dtype=torch.bfloat16, device=h.device)
    bst = _need_bf16("base_output", base_output, 2)
    _need_rows_cols("base_output", base_output, s, int(offs[-1]))
    ind, sl, nseg, hint, perm = batch_info.kernel_segments()
    check(calls().lora_expand(
        _vp(h), hst[0], _vp(weights), N, _vp(base_output), bst[0], s, L, R,
        p_offs, c, int(max_slice_size), _vp(ind), _vp(sl), nseg, _vp(perm),
        _vp(batch_info.lora_ranks), _vp(batch_info.scalings), hint, _stream(h)))
    return base_output


def lora_qkv(x, A, B, batch_info: LoRABatchInfo, slice_offsets, max_slice_size,
             base_output=None, workspace=None):
    """Stacked shrink + expand with one plan (qkv: 3 slices, gate_up: 2)."""
    xst = _need_bf16("x", x, 2)
    _need_bf16_dense("A", A, 3)
    _need_bf16_dense("B", B, 3)
    offs, p_offs = _offsets(slice_offsets)
    c = len(offs) - 1
    s, K = x.shape
    L, CR, K2 = A.shape
    _, N, R = B.shape
    if K2 != K or CR != c * R:
        raise ValueError(f"A shape {tuple(A.shape)} does not match x ({K}) and c*R ({c}*{R})")
    if s != batch_info.num_tokens:
        raise ValueError(f"x has {s} rows, the plan has {batch_info.num_tokens} tokens")
    if base_output is None:
        base_output = torch.zeros((s, int(offs[-1])), dtype=torch.bfloat16, device=x.device)
    bst = _need_bf16("base_output", base_output, 2)
    _need_rows_cols("base_output", base_output, s, int(offs[-1]))
    ind, sl, nseg, hint, perm = batch_info.kernel_segments()
    ws = workspace
    if ws is None:   # the library checks the size of a caller's workspace itself
        need = calls().lora_qkv_workspace_bytes(s, K, c, R, nseg, hint)
        ws = default_workspace(x.device, max(need, 1))
    check(calls().lora_qkv(
        x.data_ptr(), xst[0], A.data_ptr(), B.data_ptr(), N, base_output.data_ptr(),
        bst[0], s, K, L, R, p_offs, c, int(max_slice_size), ind.data_ptr(),
        sl.data_ptr(), nseg, perm.data_ptr(), batch_info.lora_ranks.data_ptr(),
        batch_info.scalings.data_ptr(), hint, ws.data_ptr(), ws.numel(), _stream(x)))
    return base_output


def lora_qkv_noalloc(x, A, B, batch_info: LoRABatchInfo, slice_offsets, max_slice_size,
                     base_output):
    """lora_qkv with the library's own device scratch instead of a workspace
    (no allocation anywhere; base_output is required).  Calls on one device
    share that scratch and must not overlap in time."""
    xst = _need_bf16("x", x, 2)
    _need_bf16_dense("A", A, 3)
    _need_bf16_dense("B", B, 3)
    offs, p_offs = _offsets(slice_offsets)
    c = len(offs) - 1
    s, K = x.shape
    L, CR, K2 = A.shape
    _, N, R = B.shape
    if K2 != K or CR != c * R:
        raise ValueError(f"A shape {tuple(A.shape)} does not match x ({K}) and c*R ({c}*{R})")
    if s != batch_info.num_tokens:
        raise ValueError(f"x has {s} rows, the plan has {batch_info.num_tokens} tokens")
    bst = _need_bf16("base_output", base_output, 2)
    _need_rows_cols("base_output", base_output, s, int(offs[-1]))
    ind, sl, nseg, hint, perm = batch_info.kernel_segments()
    check(lib().lora_qkv_noalloc(
        x.data_ptr(), xst[0], A.data_ptr(), B.data_ptr(), N, base_output.data_ptr(), bst[0], s,
        K, L, R, ctypes.cast(p_offs, _P32), c, int(max_slice_size), ind.data_ptr(),
        sl.data_ptr(), nseg, perm.data_ptr(), batch_info.lora_ranks.data_ptr(),
        batch_info.scalings.data_ptr(), hint, _stream(x)))
    return base_output


def lora_moe_route(req_seg_indptr, req_weight_indices, num_reqs, topk_ids, num_experts,
                   lora_ranks, scalings, num_loras, virtual_slots, virtual_ranks,
                   virtual_scalings):
    """Virtual experts of the MoE LoRA add from the per-request routing fields
    (all device tensors; see include/sgg_lora.h): virtual_slots (int32
    [tokens * top_k]), virtual_ranks (int32) and virtual_scalings (float32)
    [num_loras * num_experts + 1] are written on the stream."""
    def dev(name, t, dtype, n):
        if t.dtype != dtype or not t.is_cuda or not t.is_contiguous() or t.numel() < n:
            raise ValueError(f"{name} must be a contiguous {dtype} device tensor of >= {n} "
                             f"entries")
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be (num_tokens, top_k)")
    s, k = topk_ids.shape
    nv = num_loras * num_experts + 1
    dev("req_seg_indptr", req_seg_indptr, torch.int32, num_reqs + 1)
    if num_reqs:
        dev("req_weight_indices", req_weight_indices, torch.int32, num_reqs)
    dev("topk_ids", topk_ids, torch.int32, s * k)
    dev("lora_ranks", lora_ranks, torch.int32, num_loras)
    dev("scalings", scalings, torch.float32, num_loras)
    dev("virtual_slots", virtual_slots, torch.int32, s * k)
    dev("virtual_ranks", virtual_ranks, torch.int32, nv)
    dev("virtual_scalings", virtual_scalings, torch.float32, nv)
    check(lib().lora_moe_route(
        req_seg_indptr.data_ptr(), req_weight_indices.data_ptr() if num_reqs else None,
        int(num_reqs), topk_ids.data_ptr(), s, k, int(num_experts), lora_ranks.data_ptr(),
        scalings.data_ptr(), int(num_loras), virtual_slots.data_ptr(),
        virtual_ranks.data_ptr(), virtual_scalings.data_ptr(), _stream(topk_ids)))


def lora_moe_plan(req_seg_indptr, req_weight_indices, num_reqs, topk_ids, num_experts,
                  lora_ranks, scalings, num_loras, max_chunk_size, seg_capacity, device_plan,
                  device_info):
    """lora_moe_route and lora_plan_device over the copies in one launch (all
    device tensors; see include/sgg_lora.h): the copies' plan in device_plan
    (int32, lora_plan_layout(s * k, seg_capacity, s * k, L * E + 1)), the
    virtual rank / scaling tables in its regions 5 and 6, counts and status
    in device_info (int32 [8])."""
    def dev(name, t, dtype, n):
        if t.dtype != dtype or not t.is_cuda or not t.is_contiguous() or t.numel() < n:
            raise ValueError(f"{name} must be a contiguous {dtype} device tensor of >= {n} "
                             f"entries")
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be (num_tokens, top_k)")
    s, k = topk_ids.shape
    dev("req_seg_indptr", req_seg_indptr, torch.int32, num_reqs + 1)
    if num_reqs:
        dev("req_weight_indices", req_weight_indices, torch.int32, num_reqs)
    dev("topk_ids", topk_ids, torch.int32, s * k)
    dev("lora_ranks", lora_ranks, torch.int32, num_loras)
    dev("scalings", scalings, torch.float32, num_loras)
    dev("device_plan", device_plan, torch.int32, 1)
    dev("device_info", device_info, torch.int32, 8)
    check(lib().lora_moe_plan(
        req_seg_indptr.data_ptr(), req_weight_indices.data_ptr() if num_reqs else None,
        int(num_reqs), topk_ids.data_ptr(), s, k, int(num_experts), lora_ranks.data_ptr(),
        scalings.data_ptr(), int(num_loras), int(max_chunk_size), int(seg_capacity),
        device_plan.data_ptr(), 4 * device_plan.numel(), device_info.data_ptr(),
        _stream(topk_ids)))


def lora_moe_add(x, A, B, moe_info: LoRABatchInfo, top_k, out, workspace=None):
    """MoE LoRA add: out (tokens * top_k, N) += per copy t*top_k + j the LoRA
    delta of its virtual expert (include/sgg_lora.h).  x (tokens, K);
    A (num_virtual, R, K) or (L, E, R, K); B (num_virtual, N, R) or
    (L, E, N, R); moe_info: the plan of the copies (ChunkedSgmvLoRA.
    prepare_moe_lora_batch)."""
    xst = _need_bf16("x", x, 2)
    if A.dim() == 4:
        A = A.reshape(A.shape[0] * A.shape[1], A.shape[2], A.shape[3])
    if B.dim() == 4:
        B = B.reshape(B.shape[0] * B.shape[1], B.shape[2], B.shape[3])
    _need_bf16_dense("A", A, 3)
    _need_bf16_dense("B", B, 3)
    s, K = x.shape
    nv, R, K2 = A.shape
    _, N, R2 = B.shape
    if K2 != K or R2 != R or B.shape[0] != nv:
        raise ValueError(f"A {tuple(A.shape)} / B {tuple(B.shape)} do not match x ({K})")
    if s * top_k != moe_info.num_tokens:
        raise ValueError(f"x has {s} rows x top_k {top_k}, the plan has "
                         f"{moe_info.num_tokens} copies")
    ost = _need_bf16("out", out, 2)
    _need_rows_cols("out", out, s * top_k, N)
    ind, sl, nseg, hint, perm = moe_info.kernel_segments()
    ws = workspace
    if ws is None:
        need = calls().lora_qkv_workspace_bytes(s * top_k, K, 1, R, nseg, hint)
        ws = default_workspace(x.device, max(need, 1))
    check(lib().lora_moe_add(
        x.data_ptr(), xst[0], s, int(top_k), A.data_ptr(), B.data_ptr(), N, out.data_ptr(),
        ost[0], K, nv, R, ind.data_ptr(), sl.data_ptr(), nseg, perm.data_ptr(),
        moe_info.lora_ranks.data_ptr(), moe_info.scalings.data_ptr(), hint, ws.data_ptr(),
        ws.numel(), _stream(x)))
    return out


def lora_a_embedding(input_ids, weights, batch_info: LoRABatchInfo, vocab_size,
                     extra_embeddings=None, out=None):
    """LoRA-A embedding lookup: ids (s,), weights (L, R, V) -> (s, R)."""
    if input_ids.dtype is not torch.int64 or not input_ids.is_cuda:
        raise TypeError("input_ids must be an int64 tensor on a ROCm device")
    _need_bf16_dense("weights", weights, 3)
    s = input_ids.shape[0]
    L, R, V = weights.shape
    if s != batch_info.num_tokens:
        raise ValueError(f"{s} ids, the plan has {batch_info.num_tokens} tokens")
    if out is None:
        out = torch.empty((s, R), dtype=torch.bfloat16, device=weights.device)
    ost = _need_bf16("out", out, 2)
    _need_rows_cols("out", out, s, R)
    # the plan's own segments: the gather parallelises over segments, so the
    # finer partition is the faster one here
    check(calls().lora_a_embedding(
        input_ids.contiguous().data_ptr(), weights.data_ptr(), V, out.data_ptr(), ost[0],
        s, L, R, int(vocab_size), batch_info.seg_indptr.data_ptr(),
        batch_info.weight_indices.data_ptr(), batch_info.num_segments,
        batch_info.permutation.data_ptr(), batch_info.lora_ranks.data_ptr(),
        0 if extra_embeddings is None else 1, _stream(weights)))
    return out
