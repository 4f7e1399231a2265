"""lora_qkv_noalloc: lora_qkv whose workspace is the library's own device
scratch array (for callers that cannot allocate).  Called through the C ABI,
its output must equal lora_qkv's with a caller workspace bit for bit, and the
oracle within the parity tolerance, on two calls in a row (the second on a
smaller batch, after the first left its contents in the scratch); a call
whose workspace would exceed the array is refused before anything runs."""

import numpy as np
import pytest
import torch

from oracle import lora as ol
from synth import Batch, Projection, draw_batch, draw_projection, to_f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ATOL = RTOL = 1e-2


def _sgg():
    import segmented_gather_gemm_amd as sgg
    return sgg


def _pair(b, proj):
    """lora_qkv (caller workspace) and lora_qkv_noalloc on the same plan and
    inputs; returns both outputs and the oracle's."""
    sgg = _sgg()
    t = draw_projection(b, proj)
    x, A, Bw, base = (t[k].to(DEV) for k in ("x", "A", "B", "base"))
    be = sgg.ChunkedSgmvLoRA(b.num_loras, b.max_chunk_size, DEV)
    info = be.prepare_lora_batch(None if b.is_decode else b.seq_lens, b.req_slots,
                                 b.lora_ranks, b.scalings, is_decode=b.is_decode)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    y_ws = sgg.lora_qkv(x, A, Bw, info, proj.slice_offsets, proj.max_slice, base.clone(),
                        workspace=ws)
    y_na = sgg.lora_qkv_noalloc(x, A, Bw, info, proj.slice_offsets, proj.max_slice,
                                base.clone())
    torch.cuda.synchronize()
    want = ol.lora_forward(to_f64(t["x"]), to_f64(t["A"]), to_f64(t["B"]), to_f64(t["base"]),
                           b.seq_lens, b.req_slots, b.lora_ranks, b.scalings,
                           proj.slice_offsets)
    return y_ws, y_na, want


def _close(got, want, what):
    got = to_f64(got)
    assert np.isfinite(got).all(), what
    bad = np.abs(got - want) > ATOL + RTOL * np.abs(want)
    assert not bad.any(), f"{what}: {int(bad.sum())} outside tolerance"


def test_noalloc_matches_workspace_call_twice():
    # 1: the decode batch (256 tokens, split-K partials through the scratch);
    # 2: a smaller batch (tiny, 16 tokens), after the first left its contents
    for name in ("decode", "tiny"):
        b = draw_batch(name)
        proj = b.projections[0]
        y_ws, y_na, want = _pair(b, proj)
        assert torch.equal(y_na, y_ws), name
        _close(y_na, want, name)


def test_noalloc_refuses_more_than_its_scratch():
    sgg = _sgg()
    s, K, R, c = 70000, 64, 64, 2          # h alone: 70000 x 128 bf16 = 17.9 MB > 16 MiB
    b = Batch(name="big", seed=0, seq_lens=[s], req_slots=[0], is_decode=False, num_loras=1,
              lora_ranks=[R], scalings=[1.0], max_chunk_size=128,
              projections=[Projection("gate_up", K, [0, 8, 16], R)])
    be = sgg.ChunkedSgmvLoRA(1, 128, DEV)
    info = be.prepare_lora_batch(b.seq_lens, b.req_slots, b.lora_ranks, b.scalings)
    x = torch.zeros((s, K), dtype=torch.bfloat16, device=DEV)
    A = torch.zeros((1, c * R, K), dtype=torch.bfloat16, device=DEV)
    Bw = torch.zeros((1, 16, R), dtype=torch.bfloat16, device=DEV)
    base = torch.zeros((s, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sgg.SggError) as err:
        sgg.lora_qkv_noalloc(x, A, Bw, info, [0, 8, 16], 8, base)
    assert err.value.code == -3 and "scratch" in str(err.value)
    torch.cuda.synchronize()
    assert not base.any()
