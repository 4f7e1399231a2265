"""Workload definitions and seeded generators for chunked SGMV LoRA.

Five workloads, shaped like the pages' decode / prefill serving batches:

=========  ==============================================================
tiny       4 requests, lengths [3, 5, 1, 7] (16 tokens), slots [0, 1, 0, 1],
           2 adapters of rank 8, scaling 2.0, in = out = 256, one slice,
           server chunk cap 16.
decode     256 requests of one token (decode mode), 8 adapters drawn
           uniformly, rank 16, scaling 1.0, stacked qkv: in 4096,
           slice offsets [0, 4096, 5120, 6144]; chunk cap 128.
prefill    32 requests with lengths uniform in [64, 2048], 32 adapters
           drawn from a Zipf(1.1) law truncated to 32 slots, rank 64,
           scaling 1.0, gate_up: in 4096, offsets [0, 14336, 28672];
           chunk cap swept over 16 / 32 / 64 / 128.
skewed     8192 tokens: one hot adapter (slot 1) with 14 x 512 + 205 tokens
           (90 %), 819 one-token requests spread over the other 127 slots,
           request order shuffled; ranks (8, 16, 32, 64)[slot % 4] padded
           to 64 with NaN in the padding, scaling 16 / rank; o_proj
           4096 -> 4096 and down_proj 14336 -> 4096; extend mode, cap 128.
full       Llama-3-8B-shaped layer stack: 192 one-token requests plus 8
           requests of 512 tokens (4288 tokens, extend mode), 64 adapters
           drawn uniformly, rank 32, scaling 1.0; per layer qkv (c=3,
           4096 -> 6144), o (4096 -> 4096), gate_up (c=2, 4096 -> 28672),
           down (14336 -> 4096), 32 layers with distinct weights; plus the
           LoRA-A embedding gather with vocab 128256, rank 16, uniform ids.
=========  ==============================================================

Values: x and base ~ N(0, 1), A and B ~ N(0, 0.02^2), drawn as float32 and
rounded to bf16 (round to nearest even) by torch.  Every piece comes from its
own PCG64 stream keyed by (workload seed, layer, projection, tensor kind,
block), so any row block or adapter can be regenerated alone and large
tensors can be drawn in parallel.  Workload seeds are 1001..1005.

Nothing here plans a batch or multiplies a matrix.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

ROW_BLOCK = 1024          # rows per independent activation stream
KIND_X, KIND_A, KIND_B, KIND_BASE, KIND_IDS, KIND_EMB = 1, 2, 3, 4, 5, 6


@dataclass
class Projection:
    """One LoRA call: in_dim K, stacked slice offsets, padded rank R."""
    name: str
    in_dim: int
    slice_offsets: List[int]
    rank: int

    @property
    def num_slices(self):
        return len(self.slice_offsets) - 1

    @property
    def out_dim(self):
        return self.slice_offsets[-1]

    @property
    def max_slice(self):
        o = self.slice_offsets
        return max(o[i + 1] - o[i] for i in range(len(o) - 1))


@dataclass
class Batch:
    """Batch structure: what the planner and the oracle both start from."""
    name: str
    seed: int
    seq_lens: List[int]
    req_slots: List[int]
    is_decode: bool
    num_loras: int
    lora_ranks: List[int]
    scalings: List[float]
    max_chunk_size: int
    projections: List[Projection] = field(default_factory=list)
    num_layers: int = 1
    nan_padding: bool = False
    vocab_size: int = 0
    emb_rank: int = 0

    @property
    def num_tokens(self):
        return int(sum(self.seq_lens))


LLAMA_QKV = Projection("qkv", 4096, [0, 4096, 5120, 6144], 32)
LLAMA_O = Projection("o", 4096, [0, 4096], 32)
LLAMA_GATE_UP = Projection("gate_up", 4096, [0, 14336, 28672], 32)
LLAMA_DOWN = Projection("down", 14336, [0, 4096], 32)

CONFIGS = ("tiny", "decode", "prefill", "skewed", "full")
SEEDS = {"tiny": 1001, "decode": 1002, "prefill": 1003, "skewed": 1004, "full": 1005}


def _zipf_slots(rng, n, num_slots, exponent):
    """Slots 0..num_slots-1 with P(slot k-1) proportional to k^-exponent."""
    w = np.arange(1, num_slots + 1, dtype=np.float64) ** (-exponent)
    return rng.choice(num_slots, size=n, p=w / w.sum())


def draw_batch(name, max_chunk_size=None, seed=None):
    """Batch structure of one workload (lengths, slots, ranks, scalings).

    Draw order on the workload's base stream: lengths, slot assignment,
    request shuffle.
    """
    if name not in SEEDS:
        raise ValueError(f"unknown workload {name!r}")
    seed = SEEDS[name] if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "tiny":
        b = Batch(name, seed, [3, 5, 1, 7], [0, 1, 0, 1], False, 2, [8, 8],
                  [2.0, 2.0], 16, [Projection("plain", 256, [0, 256], 8)])
    elif name == "decode":
        slots = rng.integers(0, 8, size=256).tolist()
        b = Batch(name, seed, [1] * 256, slots, True, 8, [16] * 8, [1.0] * 8,
                  128, [Projection("qkv", 4096, [0, 4096, 5120, 6144], 16)])
    elif name == "prefill":
        lens = rng.integers(64, 2049, size=32).tolist()
        slots = _zipf_slots(rng, 32, 32, 1.1).tolist()
        b = Batch(name, seed, lens, slots, False, 32, [64] * 32, [1.0] * 32,
                  128, [Projection("gate_up", 4096, [0, 14336, 28672], 64)])
    elif name == "skewed":
        hot = [512] * 14 + [205]
        others = [s for s in range(128) if s != 1]
        cold = rng.choice(others, size=819).tolist()
        lens = hot + [1] * len(cold)
        slots = [1] * len(hot) + cold
        order = rng.permutation(len(lens))
        lens = [lens[i] for i in order]
        slots = [int(slots[i]) for i in order]
        ranks = [(8, 16, 32, 64)[a % 4] for a in range(128)]
        b = Batch(name, seed, lens, slots, False, 128, ranks,
                  [16.0 / r for r in ranks], 128,
                  [Projection("o_proj", 4096, [0, 4096], 64),
                   Projection("down_proj", 14336, [0, 4096], 64)],
                  nan_padding=True)
    else:  # full
        lens = [1] * 192 + [512] * 8
        slots = rng.integers(0, 64, size=len(lens)).tolist()
        order = rng.permutation(len(lens))
        lens = [lens[i] for i in order]
        slots = [int(slots[i]) for i in order]
        b = Batch(name, seed, lens, slots, False, 64, [32] * 64, [1.0] * 64,
                  128, [LLAMA_QKV, LLAMA_O, LLAMA_GATE_UP, LLAMA_DOWN],
                  num_layers=32, vocab_size=128256, emb_rank=16)
    if max_chunk_size is not None:
        b.max_chunk_size = max_chunk_size
    return b


def _bf16(arr):
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(torch.bfloat16)


def _normal_rows(key, rows, cols, std, row_lo=0, row_hi=None, threads=8):
    """Rows [row_lo, row_hi) of a (rows, cols) N(0, std^2) matrix as bf16.

    Row block b (ROW_BLOCK rows) comes from its own stream ``key + (b,)``.
    """
    row_hi = rows if row_hi is None else row_hi
    out = torch.empty((row_hi - row_lo, cols), dtype=torch.bfloat16)
    blocks = range(row_lo // ROW_BLOCK, (row_hi + ROW_BLOCK - 1) // ROW_BLOCK)

    def fill(b):
        lo, hi = b * ROW_BLOCK, min((b + 1) * ROW_BLOCK, rows)
        g = np.random.default_rng(list(key) + [b])
        vals = g.standard_normal((hi - lo, cols), dtype=np.float32) * np.float32(std)
        a, z = max(lo, row_lo), min(hi, row_hi)
        if a < z:
            out[a - row_lo:z - row_lo] = _bf16(vals[a - lo:z - lo])

    if len(blocks) > 1 and threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, blocks))
    else:
        for b in blocks:
            fill(b)
    return out


def _weights(key, num_loras, rows, cols, std, ranks, R, nan_pad, a_side, threads=8):
    """Per-adapter weight blocks: A-like (c*R, K) or B-like (N, R) per slot.

    With ``nan_pad`` the entries beyond each slot's rank (rows j >= rank of
    every R-block for A, columns j >= rank for B) hold NaN.
    """
    out = torch.empty((num_loras, rows, cols), dtype=torch.bfloat16)

    def fill(a):
        g = np.random.default_rng(list(key) + [a])
        vals = g.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
        if nan_pad:
            rho = ranks[a]
            if a_side:
                for k in range(rows // R):
                    vals[k * R + rho:(k + 1) * R, :] = np.nan
            else:
                vals[:, rho:] = np.nan
        out[a] = _bf16(vals)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(num_loras)))
    return out


def draw_projection(batch: Batch, proj: Projection, layer=0, proj_index=None,
                    parts=("x", "A", "B", "base"), rows=None):
    """Tensors of one projection call as CPU bf16 tensors.

    x (s, K), A (L, c*R, K), B (L, N, R), base (s, N).  ``rows`` = (lo, hi)
    restricts x and base to a row range (the other rows are not drawn).
    """
    if proj_index is None:
        proj_index = batch.projections.index(proj)
    key = [batch.seed, layer, proj_index]
    s = batch.num_tokens
    lo, hi = (0, s) if rows is None else rows
    c, R, K, N = proj.num_slices, proj.rank, proj.in_dim, proj.out_dim
    out = {}
    if "x" in parts:
        out["x"] = _normal_rows(key + [KIND_X], s, K, 1.0, lo, hi)
    if "A" in parts:
        out["A"] = _weights(key + [KIND_A], batch.num_loras, c * R, K, 0.02,
                            batch.lora_ranks, R, batch.nan_padding, True)
    if "B" in parts:
        out["B"] = _weights(key + [KIND_B], batch.num_loras, N, R, 0.02,
                            batch.lora_ranks, R, batch.nan_padding, False)
    if "base" in parts:
        out["base"] = _normal_rows(key + [KIND_BASE], s, N, 1.0, lo, hi)
    return out


def draw_ids(batch: Batch, vocab_size=None):
    """Token ids (s,) int64 uniform over the vocabulary."""
    V = vocab_size or batch.vocab_size or 128256
    g = np.random.default_rng([batch.seed, 0, 0, KIND_IDS])
    return torch.from_numpy(g.integers(0, V, size=batch.num_tokens).astype(np.int64))


def draw_embedding(batch: Batch, vocab_size=None, emb_rank=None):
    """Token ids (s,) int64 uniform over the vocabulary and A_emb (L, R_e, V)."""
    V = vocab_size or batch.vocab_size or 128256
    Re = emb_rank or batch.emb_rank or 16
    A_emb = _weights([batch.seed, 0, 0, KIND_EMB], batch.num_loras, Re, V, 0.02,
                     batch.lora_ranks, Re, False, True)
    return draw_ids(batch, V), A_emb


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16 (or float) tensor to a float64 NumPy array."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def rotation_batch(batch: Batch, index: int) -> Optional[Batch]:
    """An independent copy of a workload's structure for buffer rotation.

    Same shapes and distributions, drawn from seed ``seed * 1000 + index``.
    """
    return draw_batch(batch.name, batch.max_chunk_size, seed=batch.seed * 1000 + index)
