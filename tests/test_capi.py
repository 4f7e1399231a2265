"""CPU tests of the C-ABI library: it loads, exports what the header declares,
plans bit-exactly like the oracle, and rejects bad arguments on the host
before anything reaches a GPU (no compute call here needs a device)."""

import ctypes
import itertools
import os
import random
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgg_lora.h")
LIBPATH = os.path.join(ROOT, "segmented_gather_gemm_amd", "libsgg_lora.so")


def _ensure_built():
    if not os.path.exists(LIBPATH):
        import __graft_entry__
        __graft_entry__.build()


_ensure_built()

import segmented_gather_gemm_amd as sgg  # noqa: E402
from segmented_gather_gemm_amd import _lib  # noqa: E402
from oracle import plan as op  # noqa: E402
from synth import CONFIGS, draw_batch  # noqa: E402


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_\w+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared()
    assert {"lora_plan_segments", "lora_shrink", "lora_expand", "lora_qkv",
            "lora_a_embedding", "lora_last_error"} <= set(names)
    handle = ctypes.CDLL(LIBPATH)
    for name in names:
        assert hasattr(handle, name), name
    # the binding declares every exported entry point, with the same names
    assert set(names) == set(_lib.SIGNATURES)


# ------------------------------------------------------------ planner parity

def _native(lens, slots, max_loras, is_decode, cap_chunk, override=0, capacity=None):
    return sgg.lora_plan_segments(lens, slots, max_loras, is_decode, cap_chunk, override,
                                  seg_capacity=capacity)


def _compare(lens, slots, max_loras, is_decode, cap_chunk, override=0, capacity=None):
    nat = _native(lens, slots, max_loras, is_decode, cap_chunk, override, capacity)
    cap = nat["capacity"]
    ref = op.plan(lens, slots, is_decode, cap_chunk, override, capacity=cap)
    s = ref["num_tokens"]
    assert nat["num_tokens"] == s
    assert nat["chunk_size"] == ref["chunk_size"]
    assert nat["num_segments"] == ref["num_segments"]
    assert list(nat["permutation"][:s]) == ref["permutation"]
    assert list(nat["seg_indptr"][:cap + 1]) == ref["seg_indptr"]
    assert list(nat["seg_slots"][:cap]) == ref["seg_slots"]
    assert list(nat["req_seg_indptr"]) == ref["req_seg_indptr"]
    return nat


def test_plan_page_examples():
    nat = _compare([2, 1, 3], [0, 1, 0], 2, False, 128, override=3)
    assert list(nat["permutation"]) == [0, 1, 3, 4, 5, 2]
    assert nat["num_segments"] == 3
    assert list(nat["seg_indptr"][:4]) == [0, 3, 5, 6]
    assert list(nat["seg_slots"][:3]) == [0, 0, 1]


@pytest.mark.parametrize("name", CONFIGS)
def test_plan_workloads(name):
    b = draw_batch(name)
    caps = [16, 32, 64, 128] if name == "prefill" else [b.max_chunk_size]
    for cap in caps:
        _compare(None if b.is_decode else b.seq_lens, b.req_slots, b.num_loras, b.is_decode, cap)


def test_plan_exhaustive_tiny():
    for bs in range(0, 4):
        for lens in itertools.product(range(4), repeat=bs):
            for slots in itertools.product(range(3), repeat=bs):
                for override in (1, 2, 3, 0):
                    _compare(list(lens), list(slots), 3, False, 128, override)


def test_plan_random_fuzz():
    rng = random.Random(3)
    for _ in range(300):
        bs = rng.randint(0, 60)
        L = rng.randint(1, 12)
        lens = [rng.choice([0, 1, 1, 3, 16, 17, 100, 300]) for _ in range(bs)]
        slots = [rng.randrange(L) for _ in range(bs)]
        cap_chunk = rng.choice([1, 8, 16, 17, 32, 48, 64, 128, 256])
        override = rng.choice([0, 0, 0, 1, 5, 16])
        _compare(lens, slots, L, False, cap_chunk, override)


def test_plan_decode_and_padding():
    slots = [3, 1, 3, 0, 2] * 20
    _compare(None, slots, 4, True, 128)
    nat = _compare([3, 5, 1, 7], [0, 1, 0, 1], 2, False, 16, capacity=6)
    assert list(nat["seg_slots"]) == [0, 1, 0, 0, 0, 0]
    assert list(nat["seg_indptr"]) == [0, 4, 16, 16, 16, 16, 16]
    nat = _compare([], [], 4, False, 128)
    assert nat["num_segments"] == 0 and nat["num_tokens"] == 0


def test_plan_errors():
    with pytest.raises(sgg.SggError) as e:
        _native([1, 2], [0, 5], 4, False, 128)
    assert e.value.code == -3 and "req_slots[1]=5" in str(e.value)
    with pytest.raises(sgg.SggError) as e:
        _native([1, -2], [0, 1], 4, False, 128)
    assert e.value.code == -1
    with pytest.raises(sgg.SggError) as e:
        _native([1, 2], [0, 1], 4, True, 128)
    assert e.value.code == -1 and "decode" in str(e.value)
    with pytest.raises(sgg.SggError) as e:
        _native([40, 40], [0, 1], 4, False, 128, override=16, capacity=3)
    assert e.value.code == -3


def test_plan_segment_bound_holds():
    rng = random.Random(5)
    for _ in range(200):
        bs = rng.randint(1, 50)
        L = rng.randint(1, 20)
        lens = [rng.randint(0, 200) for _ in range(bs)]
        slots = [rng.randrange(L) for _ in range(bs)]
        ref = op.plan(lens, slots, False, rng.choice([16, 32, 128]))
        assert ref["num_segments"] <= sgg.lora_plan_max_segments(sum(lens), L, 16)


# ------------------------------------------------------ argument validation

L = _lib.lib()
FAKE = ctypes.c_void_p(0x10000)      # 16-byte aligned, never dereferenced on the host
NULL = ctypes.c_void_p(0)


def _shrink(**kw):
    a = dict(x=FAKE, ldx=256, A=FAKE, h=FAKE, ldh=8, s=16, K=256, L=2, c=1, R=8,
             indptr=FAKE, slots=FAKE, nseg=2, perm=FAKE, ranks=FAKE, chunk=16,
             ws=NULL, wsb=0)
    a.update(kw)
    return L.lora_shrink(a["x"], a["ldx"], a["A"], a["h"], a["ldh"], a["s"], a["K"], a["L"],
                         a["c"], a["R"], a["indptr"], a["slots"], a["nseg"], a["perm"],
                         a["ranks"], a["chunk"], a["ws"], a["wsb"], NULL)


def _expand(offs=(0, 256), **kw):
    arr = (ctypes.c_int32 * len(offs))(*offs)
    a = dict(h=FAKE, ldh=8, B=FAKE, N=256, out=FAKE, ldo=256, s=16, L=2, R=8, c=len(offs) - 1,
             maxs=256, indptr=FAKE, slots=FAKE, nseg=2, perm=FAKE, ranks=FAKE, scal=FAKE,
             chunk=16)
    a.update(kw)
    return L.lora_expand(a["h"], a["ldh"], a["B"], a["N"], a["out"], a["ldo"], a["s"], a["L"],
                         a["R"], arr, a["c"], a["maxs"], a["indptr"], a["slots"], a["nseg"],
                         a["perm"], a["ranks"], a["scal"], a["chunk"], NULL)


def _err():
    return L.lora_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(x=NULL), -1, "NULL"),
    (dict(K=0), -1, "in_dim"),
    (dict(c=0), -1, "num_slices"),
    (dict(c=9, ldh=72), -1, "num_slices"),
    (dict(ldx=128), -1, "ldx"),
    (dict(ldh=4), -1, "ldh"),
    (dict(K=252, ldx=252), -2, "multiples of 8"),
    (dict(R=12, ldh=12), -2, "multiples of 8"),
    (dict(x=ctypes.c_void_p(0x10008)), -2, "aligned"),
    (dict(indptr=NULL), -1, "plan array"),
    (dict(perm=NULL), -1, "permutation is NULL"),
    (dict(nseg=-1), -1, "num_segments"),
    (dict(L=0), -1, "num_loras"),
    (dict(chunk=0), -1, "chunk_size"),
    (dict(s=-1), -1, "s="),
    (dict(s=256, K=4096, ldx=4096, c=3, R=16, ldh=48, nseg=8, chunk=128), -3, "workspace"),
])
def test_shrink_rejects(kw, code, text):
    assert _shrink(**kw) == code
    assert text in _err()


def test_shrink_empty_is_noop():
    assert _shrink(s=0) == 0
    assert _shrink(nseg=0) == 0


@pytest.mark.parametrize("offs,kw,code,text", [
    ((0, 256), dict(out=NULL), -1, "base_output is NULL"),
    ((1, 256), {}, -1, "slice_offsets[0]"),
    ((0, 200, 100), {}, -1, "non-decreasing"),
    ((0, 256), dict(maxs=255), -1, "max_slice_size"),
    ((0, 256), dict(N=255), -1, "rows"),
    ((0, 256), dict(ldo=255), -1, "ldo"),
    ((0, 128, 256), dict(ldh=8), -1, "ldh"),
    ((0, 256), dict(R=136, ldh=136), -2, "above 128"),
    ((0, 256), dict(B=ctypes.c_void_p(0x10002)), -2, "aligned"),
    ((0, 256), dict(out=ctypes.c_void_p(0x10001)), -2, "aligned"),
    ((0, 256), dict(scal=NULL), -1, "NULL"),
    ((0,) * 10, dict(c=9, maxs=0), -1, "num_slices"),
])
def test_expand_rejects(offs, kw, code, text):
    assert _expand(offs, **kw) == code
    assert text in _err()


def test_expand_empty_is_noop():
    assert _expand(s=0) == 0
    assert _expand((0, 0)) == 0


def test_embedding_rejects():
    def emb(extra=0, **kw):
        a = dict(ids=FAKE, A=FAKE, V=1000, out=FAKE, ldo=16, s=4, L=2, R=16, vocab=1000,
                 indptr=FAKE, slots=FAKE, nseg=1, perm=FAKE, ranks=FAKE)
        a.update(kw)
        return L.lora_a_embedding(a["ids"], a["A"], a["V"], a["out"], a["ldo"], a["s"], a["L"],
                                  a["R"], a["vocab"], a["indptr"], a["slots"], a["nseg"],
                                  a["perm"], a["ranks"], extra, NULL)
    assert emb(extra=1) == -2 and "extra" in _err()
    assert emb(vocab=1001) == -1 and "vocab_size" in _err()
    assert emb(ldo=8) == -1 and "ldo" in _err()
    assert emb(ids=NULL) == -1
    assert emb(s=0) == 0


def test_plan_upload_embedding_rejects():
    """The lookup's arguments are checked before the batch is planned or
    anything enqueued; the plan's own checks follow (all on the host)."""
    C = _lib.calls()
    f = FAKE.value
    slots = np.zeros(4, np.int32)
    ranks = np.full(2, 16, np.int32)
    scal = np.ones(2, np.float32)
    info = np.zeros(6, np.int32)

    def call(staging=f, ids=f, A=f, V=1000, out=f, ldo=16, R=16, vocab=1000):
        return C.lora_plan_upload_embedding(None, slots, 4, ranks, scal, 2, 1, 128, 0, 4, 8, 4,
                                            staging, f, 1 << 16, info, None, 0, ids, A, V, out,
                                            ldo, R, vocab, None)
    assert call(R=0) == -1 and "R=0" in _err()
    assert call(vocab=1001) == -1 and "vocab_size" in _err()
    assert call(ldo=8) == -1 and "ldo" in _err()
    assert call(ids=0) == -1 and "NULL" in _err()
    assert call(out=f + 1) == -2 and "misaligned" in _err()
    assert call(staging=0) == -1 and "host_staging" in _err()


def test_qkv_rejects():
    offs = (ctypes.c_int32 * 4)(0, 4096, 5120, 6144)
    args = [FAKE, 4096, FAKE, FAKE, 6144, FAKE, 6144, 256, 4096, 8, 16, offs, 3, 4096,
            FAKE, FAKE, 8, FAKE, FAKE, FAKE, 128]
    assert L.lora_qkv(*args, NULL, 0, NULL) == -1 and "workspace" in _err()
    need = L.lora_qkv_workspace_bytes(256, 4096, 3, 16, 8, 128)
    assert need > 256 * 48 * 2
    assert L.lora_qkv(*args, FAKE, need - 1, NULL) == -3 and "workspace" in _err()


def test_moe_route_rejects():
    def route(**kw):
        a = dict(indptr=FAKE, wi=FAKE, bs=4, topk=FAKE, s=8, k=2, E=8, ranks=FAKE, scal=FAKE,
                 L=4, slots=FAKE, vr=FAKE, vs=FAKE)
        a.update(kw)
        return L.lora_moe_route(a["indptr"], a["wi"], a["bs"], a["topk"], a["s"], a["k"],
                                a["E"], a["ranks"], a["scal"], a["L"], a["slots"], a["vr"],
                                a["vs"], NULL)
    assert route(k=0) == -1 and "top_k" in _err()
    assert route(E=0) == -1 and "num_experts" in _err()
    assert route(s=-1) == -1
    assert route(indptr=NULL) == -1 and "req_seg_indptr" in _err()
    assert route(wi=NULL) == -1 and "req_weight_indices" in _err()
    assert route(topk=NULL) == -1 and "topk_ids" in _err()
    assert route(s=1 << 30, k=4) == -2 and "int32" in _err()
    assert route(L=1 << 20, E=1 << 12) == -2 and "int32" in _err()


def test_moe_plan_rejects():
    """Host checks of the one-launch routing + plan: the device planner's
    limits, the plan buffer's size, NULL pointers (nothing is enqueued)."""
    def plan(tokens=4, k=2, E=2, L=2, buf=FAKE, nbytes=1 << 16, info=FAKE, topk=FAKE):
        return L_.lora_moe_plan(FAKE, FAKE, 2, topk, tokens, k, E, FAKE, FAKE, L, 128, 16, buf,
                                nbytes, info, NULL)
    L_ = L
    assert plan(tokens=2049) == -2 and "copies" in _err()
    assert plan(E=512) == -2 and "1024" in _err()
    assert plan(nbytes=64) == -3 and "plan buffer" in _err()
    assert plan(buf=NULL) == -1
    assert plan(info=NULL) == -1
    assert plan(topk=NULL) == -1 and "topk_ids" in _err()
    assert plan(k=0) == -1


def test_moe_add_rejects():
    def add(ws=NULL, wsb=0, **kw):
        a = dict(x=FAKE, ldx=512, s=64, k=2, A=FAKE, B=FAKE, N=256, out=FAKE, ldo=256, K=512,
                 nv=32, R=16, indptr=FAKE, slots=FAKE, nseg=8, perm=FAKE, ranks=FAKE,
                 scal=FAKE, chunk=16)
        a.update(kw)
        return L.lora_moe_add(a["x"], a["ldx"], a["s"], a["k"], a["A"], a["B"], a["N"],
                              a["out"], a["ldo"], a["K"], a["nv"], a["R"], a["indptr"],
                              a["slots"], a["nseg"], a["perm"], a["ranks"], a["scal"],
                              a["chunk"], ws, wsb, NULL)
    assert add(k=0) == -1 and "top_k" in _err()
    assert add(s=1 << 30, k=4) == -2 and "int32" in _err()
    assert add() == -1 and "workspace" in _err()
    assert add(ws=FAKE, wsb=1 << 30, ldo=128) == -1 and "ldo" in _err()
    assert add(ws=FAKE, wsb=1 << 30, ldx=256) == -1 and "ldx" in _err()


def test_workspace_sizes():
    # decode shapes split K across workgroups and need scratch; prefill shapes
    # do not, unless the segment-pair tiles (K in two ranges) are asked for
    assert L.lora_shrink_workspace_bytes(256, 4096, 3, 16, 8, 128) > 0
    assert L.lora_shrink_workspace_bytes(33792, 4096, 2, 64, 300, 128) == 0
    old = L.lora_set_option(b"shrink_pair_tiles", 1)
    try:
        assert L.lora_shrink_workspace_bytes(33792, 4096, 2, 64, 300, 128) >= 2 * 33792 * 128 * 4
        assert L.lora_shrink_workspace_bytes(33792, 4096, 2, 32, 300, 128) == 0
    finally:
        L.lora_set_option(b"shrink_pair_tiles", old)
    assert L.lora_shrink_workspace_bytes(0, 4096, 3, 16, 8, 128) == 0
    # short segments with c*R <= 32 and a long K: 64-token tiles with K split
    # in ranges of 1792 (8 for the full-layer down_proj), the split-K
    # counters then the f32 partials [8][s][c*R]
    s, cr = 4288, 32
    assert (L.lora_shrink_workspace_bytes(s, 14336, 1, 32, 93, 128)
            == 65536 + (8 * s * cr * 4 + 255) // 256 * 256)
    # ... but not with K = 4096 (one range) nor with c*R = 64 (GEMM tiles)
    assert L.lora_shrink_workspace_bytes(s, 4096, 1, 32, 93, 128) == 0
    assert L.lora_shrink_workspace_bytes(8192, 14336, 1, 64, 185, 128) == 0
    # decode-shaped qkv (c*R = 48) of 1024 / 2048 tokens over 8 adapters:
    # 16-token tiles over all 48 rank rows with K in 4 / 2 ranges; 256 and
    # 4096 tokens keep 16 x 16 tiles in 4 ranges and 32 x 16 tiles over all K
    assert L.lora_shrink_workspace_bytes(1024, 4096, 3, 16, 11, 128) == 65536 + 4 * 1024 * 48 * 4
    assert L.lora_shrink_workspace_bytes(2048, 4096, 3, 16, 20, 128) == 65536 + 2 * 2048 * 48 * 4
    assert L.lora_shrink_workspace_bytes(256, 4096, 3, 16, 8, 40) == 65536 + 4 * 256 * 48 * 4
    assert L.lora_shrink_workspace_bytes(4096, 4096, 3, 16, 36, 128) == 0


def test_error_is_thread_local():
    import threading
    assert _shrink(K=0) == -1
    seen = []
    t = threading.Thread(target=lambda: seen.append(_err()))
    t.start()
    t.join()
    assert seen == [""]
    assert "in_dim" in _err()


def test_library_never_imports_oracle():
    imp_oracle = re.compile(r"^\s*(from|import)\s+oracle\b", re.M)
    imp_lib = re.compile(r"^\s*(from|import)\s+(segmented_gather_gemm_amd|synth)\b", re.M)
    pkg = os.path.join(ROOT, "segmented_gather_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                assert not imp_oracle.search(open(os.path.join(dirpath, f)).read()), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            assert not imp_lib.search(open(os.path.join(ROOT, "oracle", f)).read()), f


def test_np_dtypes_roundtrip():
    nat = _native(np.array([2, 3], np.int64), np.array([1, 0], np.int64), 2, False, 16)
    assert list(nat["permutation"][:5]) == [2, 3, 4, 0, 1]


def test_plan_layout_regions():
    """lora_plan_layout: 10 regions (plan, routing, tables, work segments,
    work permutation), 64-element aligned, in the documented order and sizes."""
    lib = _lib.lib()
    offs = (ctypes.c_int64 * 10)()
    total = lib.lora_plan_layout(300, 40, 20, 8, offs)
    sizes = [300, 41, 40, 21, 20, 8, 8, 41, 40, 300]
    pos = 0
    for i, n in enumerate(sizes):
        assert offs[i] == pos, i
        pos += (n + 63) // 64 * 64
    assert total == pos
    assert lib.lora_plan_layout(-1, 0, 0, 1, None) == -1


def _lm_head_native(lens, slots, L, cap, override=0):
    got = sgg.lora_plan_lm_head(lens, slots, L, cap, override)
    n = got["num_segments"]
    return {"permutation": got["permutation"].tolist(),
            "seg_indptr": got["seg_indptr"][:n + 1].tolist(),
            "seg_slots": got["seg_slots"][:n].tolist(), "num_segments": n,
            "chunk_size": got["chunk_size"], "num_tokens": got["num_tokens"]}


def test_lm_head_planner_matches_oracle_exhaustive():
    """Every tiny pruned batch (bs <= 4, lengths 0..3, slots 0..2) and forced
    chunks: the native lm_head planner equals the oracle bit for bit."""
    for bs in range(0, 5):
        for lens in itertools.product(range(0, 4), repeat=bs):
            for slots in itertools.product(range(0, 3), repeat=bs):
                for override in (0, 1, 2, 3):
                    want = op.lm_head_plan(list(lens), list(slots), 128, override)
                    got = _lm_head_native(list(lens), list(slots), 3, 128, override)
                    for k in got:
                        assert got[k] == want[k], (lens, slots, override, k)


def test_lm_head_planner_matches_oracle_random():
    rng = random.Random(11)
    for _ in range(300):
        bs = rng.randint(1, 64)
        lens = [rng.choice([0, 1, 1, 1, 3, 20, 150, 700]) for _ in range(bs)]
        slots = [rng.randrange(6) for _ in range(bs)]
        cap = rng.choice([8, 16, 32, 64, 128, 256])
        want = op.lm_head_plan(lens, slots, cap)
        got = _lm_head_native(lens, slots, 6, cap)
        for k in got:
            assert got[k] == want[k], k


def test_lm_head_planner_errors():
    with pytest.raises(sgg.SggError):
        sgg.lora_plan_lm_head([1, -1], [0, 0], 2, 128)
    with pytest.raises(sgg.SggError):
        sgg.lora_plan_lm_head([1, 1], [0, 2], 2, 128)     # slot outside [0, 2)
    with pytest.raises(sgg.SggError):
        sgg.lora_plan_lm_head([5, 5], [0, 1], 2, 128, seg_capacity=1)



# ------------------------------------------------------ CPython call module

def _header_signature(name):
    """'p' / 'l' / 'i' per parameter of `name` as declared in the header."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    sig = ""
    for param in m.group(1).split(","):
        param = param.strip()
        if "*" in param:
            sig += "p"
        elif param.startswith("int64_t"):
            sig += "l"
        elif param.startswith("int32_t"):
            sig += "i"
        else:
            raise AssertionError(f"{name}: unexpected parameter {param!r}")
    return sig


def test_call_module_signatures_match_header():
    C = _lib.calls()
    assert set(C.SIGNATURES) == {"lora_plan_max_segments", "lora_plan_upload", "lora_plan_device",
                                 "lora_plan_upload_embedding",
                                 "lora_plan_lm_head_upload", "lora_shrink_workspace_bytes",
                                 "lora_qkv_workspace_bytes", "lora_shrink", "lora_expand",
                                 "lora_qkv", "lora_a_embedding"}
    for name, sig in C.SIGNATURES.items():
        assert sig == _header_signature(name), name
        assert callable(getattr(C, name)), name
        with pytest.raises(TypeError, match=f"takes {len(sig)} arguments"):
            getattr(C, name)(*([0] * (len(sig) + 1)))


def test_call_module_argument_checks():
    C = _lib.calls()
    assert C.lora_plan_max_segments(4096, 8, 16) == L.lora_plan_max_segments(4096, 8, 16)
    assert C.lora_plan_max_segments(np.int64(4096), np.int32(8), 16) == \
        L.lora_plan_max_segments(4096, 8, 16)
    with pytest.raises(OverflowError):
        C.lora_plan_max_segments(10, 1 << 31, 16)
    with pytest.raises(TypeError):
        C.lora_plan_max_segments(10.5, 8, 16)
    with pytest.raises(TypeError):
        C.lora_shrink_workspace_bytes(256, 4096, 3, 16, 8, "128")
    for args in [(256, 4096, 3, 16, 8, 128), (33792, 4096, 2, 64, 300, 128), (0, 4096, 3, 16, 8, 128)]:
        assert C.lora_shrink_workspace_bytes(*args) == L.lora_shrink_workspace_bytes(*args)
        assert C.lora_qkv_workspace_bytes(*args) == L.lora_qkv_workspace_bytes(*args)


def _as_int(v):
    return v.value or 0 if isinstance(v, ctypes.c_void_p) else v


@pytest.mark.parametrize("kw", [dict(x=NULL), dict(K=0), dict(ldh=4), dict(indptr=NULL),
                                dict(x=ctypes.c_void_p(0x10008)), dict(s=0)])
def test_call_module_shrink_same_status(kw):
    """The call module passes every argument through unchanged: the library
    returns the same status and message as through ctypes."""
    a = dict(x=FAKE, ldx=256, A=FAKE, h=FAKE, ldh=8, s=16, K=256, L=2, c=1, R=8,
             indptr=FAKE, slots=FAKE, nseg=2, perm=FAKE, ranks=FAKE, chunk=16, ws=NULL, wsb=0)
    a.update(kw)
    rc = _shrink(**kw)
    msg = _err()
    v = [_as_int(a[k]) for k in ("x", "ldx", "A", "h", "ldh", "s", "K", "L", "c", "R", "indptr",
                                 "slots", "nseg", "perm", "ranks", "chunk", "ws", "wsb")]
    assert _lib.calls().lora_shrink(*v, None) == rc
    if rc:
        assert _err() == msg


def test_call_module_qkv_and_embedding_same_status():
    C = _lib.calls()
    offs = np.array([0, 4096, 5120, 6144], np.int32)
    f = FAKE.value
    args = [f, 4096, f, f, 6144, f, 6144, 256, 4096, 8, 16, offs.ctypes.data, 3, 4096,
            f, f, 8, f, f, f, 128]
    assert C.lora_qkv(*args, 0, 0, 0) == -1 and "workspace" in _err()
    need = C.lora_qkv_workspace_bytes(256, 4096, 3, 16, 8, 128)
    assert C.lora_qkv(*args, f, need - 1, 0) == -3 and "workspace" in _err()
    emb = [f, f, 1000, f, 16, 4, 2, 16, 1000, f, f, 1, f, f]
    assert C.lora_a_embedding(*emb, 1, None) == -2 and "extra" in _err()
    assert C.lora_a_embedding(*emb[:8], 1001, *emb[9:], 0, None) == -1 and "vocab_size" in _err()


def test_call_module_takes_contiguous_host_buffers():
    """A NumPy array passed for a host pointer stands for its first byte; a
    non-contiguous one is refused before the library is called."""
    C = _lib.calls()
    f = FAKE.value
    offs = np.array([0, 4096, 5120, 6144], np.int32)
    head = [f, 4096, f, f, 6144, f, 6144, 256, 4096, 8, 16]
    tail = [3, 4096, f, f, 8, f, f, f, 128, 0, 0, 0]
    assert C.lora_qkv(*head, offs, *tail) == -1 and "workspace" in _err()
    bad = np.array([0, 4096, 4097, 5120, 5121, 6144, 6145, 6146], np.int32)[::2]
    with pytest.raises((BufferError, ValueError, TypeError)):
        C.lora_qkv(*head, bad, *tail)
    # the library reads the offsets from the buffer (rejected before any launch)
    exp = [f, 8, f, 256, f, 256, 16, 2, 8]
    rest = [f, f, 2, f, f, f, 16, 0]
    assert C.lora_expand(*exp, np.array([0, 200, 100], np.int32), 2, 256, *rest) == -1
    assert "non-decreasing" in _err()
    assert C.lora_expand(*exp, np.array([1, 256], np.int32), 1, 256, *rest) == -1
    assert "slice_offsets[0]" in _err()


def test_batch_arrays_rejects_mismatched_lengths():
    """prepare_lora_batch's host arrays are checked before the native planner
    reads seq_lens[r] for every request r: a shorter seq_lens would be a host
    over-read, a longer one would drop tokens from the plan."""
    from segmented_gather_gemm_amd.backend import batch_arrays
    ranks, scal = [8] * 4, [1.0] * 4
    with pytest.raises(ValueError):
        batch_arrays([1, 2], [0, 1, 2], ranks, scal, 4)
    with pytest.raises(ValueError):
        batch_arrays([1, 2, 3, 4], [0, 1, 2], ranks, scal, 4)
    with pytest.raises(ValueError):
        batch_arrays(None, [0], [8] * 3, scal, 4)
    with pytest.raises(ValueError):
        batch_arrays([[1, 2]], [[0, 1]], ranks, scal, 4)
    lens, slots, r, sc, s = batch_arrays([1, 2, 3], [0, 1, 2], ranks, scal, 4)
    assert s == 6 and lens.dtype == np.int32 and sc.dtype == np.float32
    lens, slots, r, sc, s = batch_arrays(None, [3, 1], ranks, scal, 4)
    assert lens is None and s == 2
