"""Pins for the oracle: it is checked against things other than itself.

* values printed on the chunked_backend.py page (worked examples) and a hand
  example derived from the definitions (tests/golden/);
* closed forms (merged dense weight, the textbook single-adapter product);
* brute force in plain Python loops on tiny inputs;
* invariants (request order, request merging, zero adapters, rank padding);
* library routines the planner's steps reduce to (stable argsort);
* planted mistakes: plausible bugs written into a copy of the oracle must be
  caught by the pins above.
"""

import itertools
import json
import os
import random

import numpy as np
import pytest

from oracle import lora as ol
from oracle import plan as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- planner

def test_plan_page_permutation_example():
    ex = _load("plan_worked_examples.json")["permutation_example"]
    rows = op.token_slots(ex["seq_lens"], ex["seq_weight_indices"])
    assert rows == ex["row_weight_indices"]
    perm, sorted_slots = op.gather_permutation(rows)
    assert perm == ex["permutation"]
    assert sorted_slots == ex["weights_reordered"]


def test_plan_page_segments_example():
    ex = _load("plan_worked_examples.json")["segments_example"]
    seg_slots, indptr = op.segments(ex["weights_reordered"], ex["chunk_size"])
    assert seg_slots == ex["weight_indices"]
    assert indptr == ex["seg_indptr"]


def test_plan_page_examples_end_to_end():
    ex = _load("plan_worked_examples.json")
    p = op.plan(ex["permutation_example"]["seq_lens"],
                ex["permutation_example"]["seq_weight_indices"], False, 128,
                chunk_override=ex["segments_example"]["chunk_size"])
    assert p["permutation"] == ex["permutation_example"]["permutation"]
    assert p["seg_slots"] == ex["segments_example"]["weight_indices"]
    assert p["seg_indptr"] == ex["segments_example"]["seg_indptr"]


def test_plan_tiny_hand_derived():
    ex = _load("plan_worked_examples.json")["tiny_plan_hand_derived"]
    p = op.plan(ex["seq_lens"], ex["req_slots"], ex["is_decode"], ex["max_chunk_size"])
    for key in ("chunk_size", "permutation", "seg_indptr", "seg_slots", "req_seg_indptr"):
        assert p[key] == ex[key], key


# chunk size table: rows = server cap, columns = token counts at the
# heuristic's thresholds (values worked by hand from the rule on the
# chunked_backend.py page, _determine_chunk_size_for_tokens)
CHUNK_TABLE_TOKENS = [0, 1, 63, 64, 255, 256, 4288]
CHUNK_TABLE = {
    1: [16, 16, 16, 16, 16, 16, 16],
    8: [16, 16, 16, 16, 16, 16, 16],
    16: [16, 16, 16, 16, 16, 16, 16],
    17: [16, 16, 16, 17, 17, 17, 17],
    32: [16, 16, 16, 32, 32, 32, 32],
    48: [16, 16, 16, 32, 32, 48, 48],
    64: [16, 16, 16, 32, 32, 64, 64],
    128: [16, 16, 16, 32, 32, 128, 128],
    256: [16, 16, 16, 32, 32, 128, 128],
}


@pytest.mark.parametrize("cap", sorted(CHUNK_TABLE))
def test_chunk_size_table(cap):
    got = [op.chunk_size_for_tokens(n, cap) for n in CHUNK_TABLE_TOKENS]
    assert got == CHUNK_TABLE[cap]


def test_chunk_size_properties():
    for cap in range(1, 300, 7):
        prev = 0
        for n in range(0, 600, 3):
            c = op.chunk_size_for_tokens(n, cap)
            assert c >= op.MIN_CHUNK_SIZE
            assert c <= max(op.MIN_CHUNK_SIZE, cap)
            assert c >= prev          # never shrinks as the batch grows
            prev = c


def test_chunk_size_mode():
    # decode mode keys the rule on the batch size, extend mode on tokens
    lens = [100, 100, 100]
    assert op.plan(lens, [0, 0, 0], False, 128)["chunk_size"] == 128
    assert op.plan(None, [0] * 70, True, 128)["chunk_size"] == 32
    assert op.plan([5, 5], [0, 1], False, 128)["chunk_size"] == 16


def _check_plan_invariants(seq_lens, req_slots, p):
    rows = op.token_slots(seq_lens, req_slots)
    s = len(rows)
    perm = p["permutation"]
    chunk = p["chunk_size"]
    n_seg = p["num_segments"]
    indptr = p["seg_indptr"][:n_seg + 1]
    seg_slots = p["seg_slots"][:n_seg]
    assert sorted(perm) == list(range(s))                   # bijection
    # agrees with library stable sorts
    assert perm == [int(i) for i in np.argsort(np.asarray(rows, dtype=np.int64), kind="stable")]
    assert perm == sorted(range(s), key=lambda t: rows[t])
    assert indptr[0] == 0 and indptr[-1] == s
    assert all(seg_slots[i] <= seg_slots[i + 1] for i in range(n_seg - 1))
    per_slot = {}
    for i in range(n_seg):
        lo, hi = indptr[i], indptr[i + 1]
        assert 1 <= hi - lo <= chunk
        toks = perm[lo:hi]
        assert all(rows[t] == seg_slots[i] for t in toks)      # one slot per segment
        assert toks == sorted(toks)                             # stable inside the slot
        per_slot.setdefault(seg_slots[i], []).append(hi - lo)
    for slot, lens in per_slot.items():
        assert all(length == chunk for length in lens[:-1])    # remainder last
        assert sum(lens) == rows.count(slot)
    assert n_seg == sum(-(-rows.count(a) // chunk) for a in set(rows))
    cum = [0]
    for length in seq_lens:
        cum.append(cum[-1] + length)
    assert p["req_seg_indptr"] == cum


def test_plan_brute_force_tiny():
    """Every batch of <= 3 requests, lengths 0..3, slots 0..2, several chunks."""
    count = 0
    for bs in range(0, 4):
        for lens in itertools.product(range(4), repeat=bs):
            for slots in itertools.product(range(3), repeat=bs):
                for chunk in (1, 2, 3, 16):
                    p = op.plan(list(lens), list(slots), False, 128, chunk_override=chunk)
                    _check_plan_invariants(list(lens), list(slots), p)
                    count += 1
    assert count > 1000


def test_plan_random_invariants():
    rng = random.Random(7)
    for _ in range(200):
        bs = rng.randint(0, 40)
        lens = [rng.choice([0, 1, 1, 2, 5, 17, 40, 130]) for _ in range(bs)]
        slots = [rng.randint(0, 9) for _ in range(bs)]
        cap = rng.choice([8, 16, 32, 48, 64, 128])
        p = op.plan(lens, slots, False, cap)
        assert p["chunk_size"] == op.chunk_size_for_tokens(sum(lens), cap)
        _check_plan_invariants(lens, slots, p)


def test_plan_graph_padding():
    p = op.plan([3, 5, 1, 7], [0, 1, 0, 1], False, 16, capacity=6)
    assert p["num_segments"] == 2
    assert p["seg_slots"] == [0, 1, 0, 0, 0, 0]
    assert p["seg_indptr"] == [0, 4, 16, 16, 16, 16, 16]
    with pytest.raises(ValueError):
        op.plan([3, 5, 1, 7], [0, 1, 0, 1], False, 16, capacity=1)


def test_plan_empty_and_decode():
    p = op.plan([], [], False, 128)
    assert p["num_segments"] == 0 and p["seg_indptr"] == [0] and p["permutation"] == []
    p = op.plan(None, [2, 0, 2, 1], True, 128)
    assert p["permutation"] == [1, 3, 0, 2]
    assert p["req_seg_indptr"] == [0, 1, 2, 3, 4]
    with pytest.raises(ValueError):
        op.plan([2, 1], [0, 1], True, 128)


# -------------------------------------------------------------- math oracle

def _hand():
    ex = _load("lora_hand_example.json")
    arr = {k: np.asarray(ex[k], dtype=np.float64)
           for k in ("x", "A", "B", "base", "h", "y", "A_emb", "e")}
    return ex, arr


def test_hand_example_shrink_expand():
    ex, a = _hand()
    h = ol.shrink(a["x"], a["A"], ex["seq_lens"], ex["req_slots"], ex["lora_ranks"],
                  ex["num_slices"])
    np.testing.assert_array_equal(h, a["h"])
    y = ol.expand(h, a["B"], a["base"], ex["seq_lens"], ex["req_slots"],
                  ex["lora_ranks"], ex["scalings"], ex["slice_offsets"])
    np.testing.assert_array_equal(y, a["y"])
    y2 = ol.lora_forward(a["x"], a["A"], a["B"], a["base"], ex["seq_lens"],
                         ex["req_slots"], ex["lora_ranks"], ex["scalings"],
                         ex["slice_offsets"])
    np.testing.assert_array_equal(y2, a["y"])
    # sampled rows give the same rows
    rows = [2, 0]
    y3 = ol.lora_forward(a["x"], a["A"], a["B"], a["base"][rows], ex["seq_lens"],
                         ex["req_slots"], ex["lora_ranks"], ex["scalings"],
                         ex["slice_offsets"], rows=rows)
    np.testing.assert_array_equal(y3, a["y"][rows])


def test_hand_example_embedding():
    ex, a = _hand()
    e = ol.embedding_a(ex["input_ids"], a["A_emb"], ex["seq_lens"], ex["req_slots"],
                       ex["lora_ranks"], ex["vocab_size"])
    np.testing.assert_array_equal(e, a["e"])


def _random_case(rng, bs=5, L=3, c=2, R=4, K=7, widths=(5, 3), extra=2, ranks=None):
    lens = [int(v) for v in rng.integers(0, 4, size=bs)]
    slots = [int(v) for v in rng.integers(0, L, size=bs)]
    s = sum(lens)
    offs = [0]
    for w in widths:
        offs.append(offs[-1] + w)
    N = offs[-1]
    ranks = [int(v) for v in rng.integers(0, R + 1, size=L)] if ranks is None else ranks
    scal = [float(v) for v in rng.uniform(-2, 2, size=L)]
    x = rng.standard_normal((s, K))
    A = rng.standard_normal((L, c * R, K))
    B = rng.standard_normal((L, N, R))
    base = rng.standard_normal((s, N + extra))
    return dict(lens=lens, slots=slots, ranks=ranks, scal=scal, offs=offs, x=x, A=A,
                B=B, base=base, c=c, R=R)


def _brute(case):
    """Plain-Python loops straight from the per-token definition."""
    lens, slots, ranks, scal = case["lens"], case["slots"], case["ranks"], case["scal"]
    x, A, B, base, offs, c, R = (case[k] for k in ("x", "A", "B", "base", "offs", "c", "R"))
    tok_req = []
    for r, n in enumerate(lens):
        tok_req += [r] * n
    s, K = x.shape
    y = [[float(v) for v in row] for row in base]
    for t in range(s):
        a = slots[tok_req[t]]
        rho = ranks[a]
        h = [0.0] * (c * R)
        for k in range(c):
            for j in range(rho):
                acc = 0.0
                for q in range(K):
                    acc += A[a][k * R + j][q] * x[t][q]
                h[k * R + j] = acc
        for k in range(c):
            for n in range(offs[k], offs[k + 1]):
                acc = 0.0
                for j in range(rho):
                    acc += B[a][n][j] * h[k * R + j]
                y[t][n] += scal[a] * acc
    return np.array(y).reshape(base.shape)


def _forward(case, rows=None):
    base = case["base"] if rows is None else case["base"][rows]
    return ol.lora_forward(case["x"], case["A"], case["B"], base, case["lens"],
                           case["slots"], case["ranks"], case["scal"], case["offs"],
                           rows=rows)


def test_brute_force_tiny_random():
    rng = np.random.default_rng(11)
    for _ in range(30):
        case = _random_case(rng)
        np.testing.assert_allclose(_forward(case), _brute(case), rtol=1e-12, atol=1e-12)


def test_merged_dense_closed_form():
    rng = np.random.default_rng(12)
    for _ in range(10):
        case = _random_case(rng, bs=6, L=4, c=3, R=5, K=11, widths=(6, 2, 4))
        y = _forward(case)
        tok_req = np.repeat(np.arange(len(case["lens"])), case["lens"])
        N = case["offs"][-1]
        for t in range(len(tok_req)):
            a = case["slots"][tok_req[t]]
            W = ol.merged_dense_weight(case["A"], case["B"], a, case["ranks"][a],
                                       case["scal"][a], case["offs"])
            want = case["base"][t].copy()
            want[:N] += W @ case["x"][t]
            np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-12)


def test_textbook_single_adapter():
    """One request on one full-rank adapter, one slice: base + s*(x A^T) B^T."""
    rng = np.random.default_rng(13)
    s, K, R, N = 9, 13, 4, 10
    x = rng.standard_normal((s, K))
    A = rng.standard_normal((2, R, K))
    B = rng.standard_normal((2, N, R))
    base = rng.standard_normal((s, N))
    y = ol.lora_forward(x, A, B, base, [s], [1], [0, R], [0.0, 0.75], [0, N])
    np.testing.assert_allclose(y, base + 0.75 * (x @ A[1].T) @ B[1].T, rtol=1e-12)


def test_invariance_request_order_and_merge():
    rng = np.random.default_rng(14)
    case = _random_case(rng, bs=8, L=3)
    y = _forward(case)
    cum = np.concatenate([[0], np.cumsum(case["lens"])])
    order = rng.permutation(len(case["lens"]))
    shuffled = dict(case)
    shuffled["lens"] = [case["lens"][i] for i in order]
    shuffled["slots"] = [case["slots"][i] for i in order]
    tok = np.concatenate([np.arange(cum[i], cum[i + 1]) for i in order]).astype(np.int64)
    shuffled["x"] = case["x"][tok]
    shuffled["base"] = case["base"][tok]
    np.testing.assert_allclose(_forward(shuffled), y[tok], rtol=1e-12, atol=1e-12)
    # merge every pair of adjacent requests that share a slot
    lens, slots = [], []
    for n, a in zip(case["lens"], case["slots"]):
        if slots and slots[-1] == a:
            lens[-1] += n
        else:
            lens.append(n)
            slots.append(a)
    merged = dict(case, lens=lens, slots=slots)
    np.testing.assert_allclose(_forward(merged), y, rtol=1e-12, atol=1e-12)


def test_zero_adapter_rank_zero_and_scaling_zero():
    rng = np.random.default_rng(15)
    case = _random_case(rng, bs=6, L=3, ranks=[0, 3, 4])
    case["A"][2] = 0.0
    case["scal"][1] = 0.0
    y = _forward(case)
    # every slot is a no-op here: rank 0 (slot 0), scaling 0 (slot 1), zero A (slot 2)
    np.testing.assert_array_equal(y, case["base"])


def test_rank_padding_never_read():
    rng = np.random.default_rng(16)
    case = _random_case(rng, bs=6, L=3, ranks=[1, 2, 4])
    y = _forward(case)
    c, R = case["c"], case["R"]
    for a, rho in enumerate(case["ranks"]):
        for k in range(c):
            case["A"][a, k * R + rho:(k + 1) * R, :] = np.nan
        case["B"][a, :, rho:] = np.nan
    y_nan = _forward(case)
    assert np.isfinite(y_nan).all()
    np.testing.assert_array_equal(y_nan, y)
    # columns beyond the last slice keep base
    N = case["offs"][-1]
    np.testing.assert_array_equal(y[:, N:], case["base"][:, N:])


def test_missing_base_is_zero():
    rng = np.random.default_rng(17)
    case = _random_case(rng, extra=0)
    h = ol.shrink(case["x"], case["A"], case["lens"], case["slots"], case["ranks"], case["c"])
    y0 = ol.expand(h, case["B"], None, case["lens"], case["slots"], case["ranks"],
                   case["scal"], case["offs"])
    y = ol.expand(h, case["B"], case["base"], case["lens"], case["slots"], case["ranks"],
                  case["scal"], case["offs"])
    np.testing.assert_allclose(y0 + case["base"], y, rtol=1e-12, atol=1e-12)


def test_embedding_brute_force_and_edges():
    rng = np.random.default_rng(18)
    L, Re, V = 3, 4, 9
    lens = [2, 0, 3, 1]
    slots = [2, 1, 0, 2]
    ranks = [4, 2, 0]
    A_emb = rng.standard_normal((L, Re, V))
    ids = [0, 8, 9, -1, 3, 5]      # 9 and -1 lie outside the vocabulary
    e = ol.embedding_a(ids, A_emb, lens, slots, ranks, V)
    tok_req = [0, 0, 2, 2, 2, 3]
    for t in range(6):
        a = slots[tok_req[t]]
        for j in range(Re):
            v = ids[t]
            want = A_emb[a, j, v] if (j < ranks[a] and 0 <= v < V) else 0.0
            assert e[t, j] == want
    # for full-rank slots and in-vocabulary ids it is a column gather of A_emb
    full = ol.embedding_a([4, 7], A_emb, [2], [0], ranks, V)
    np.testing.assert_array_equal(full, A_emb[0][:, [4, 7]].T)


# ------------------------------------------------------- planted mistakes

MUTANTS = {
    "scaling dropped": [
        ("y[pos, offs[k]:offs[k + 1]] += sigma * (hk @ Bk.T)",
         "y[pos, offs[k]:offs[k + 1]] += (hk @ Bk.T)")],
    "base not added": [
        ("y = np.zeros((len(rows), width)) if base is None else np.array(base, dtype=np.float64)",
         "y = np.zeros((len(rows), width))")],
    "h block index uses rank": [
        ("hk = h[pos, k * R:k * R + rho]", "hk = h[pos, k * rho:k * rho + rho]")],
    "B rank padding read": [
        ("Bk = B[a, offs[k]:offs[k + 1], :rho]", "Bk = B[a, offs[k]:offs[k + 1], :]"),
        ("hk = h[pos, k * R:k * R + rho]", "hk = h[pos, k * R:(k + 1) * R]")],
    "A rank padding read": [
        ("Ak = A[a, k * R:k * R + rho, :]", "Ak = A[a, k * R:(k + 1) * R, :]"),
        ("h[pos, k * R:k * R + rho] = xt @ Ak.T", "h[pos, k * R:(k + 1) * R] = xt @ Ak.T")],
    "slot of neighbouring request": [
        ("a = int(req_slots[r])\n        rho = min(int(lora_ranks[a]), R)\n        if rho <= 0:\n            continue\n        xt",
         "a = int(req_slots[(r + 1) % len(req_slots)])\n        rho = min(int(lora_ranks[a]), R)\n        if rho <= 0:\n            continue\n        xt")],
    "slice rows from slice zero": [
        ("Ak = A[a, k * R:k * R + rho, :]", "Ak = A[a, 0:rho, :]")],
    "B rows shifted by slice index": [
        ("Bk = B[a, offs[k]:offs[k + 1], :rho]", "Bk = B[a, offs[k] - k:offs[k + 1] - k, :rho]")],
    "tokens assigned to requests in reverse": [
        ("return np.repeat(np.arange(len(seq_lens), dtype=np.int64), seq_lens)",
         "return np.repeat(np.arange(len(seq_lens), dtype=np.int64)[::-1], seq_lens)")],
    "embedding ignores rank": [
        ("out[p, :rho] = A_emb[a, :rho, v]", "out[p, :] = A_emb[a, :, v]")],
    "embedding wraps out-of-vocab ids": [
        ("if 0 <= v < vocab_size:", "v = v % vocab_size\n            if True:")],
}


def _mutant_module(edits):
    import types
    src = open(ol.__file__).read()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    """Run the hand example, brute force and NaN-padding pins against a module."""
    try:
        ex, a = _hand()
        h = mod.shrink(a["x"], a["A"], ex["seq_lens"], ex["req_slots"], ex["lora_ranks"],
                       ex["num_slices"])
        y = mod.expand(h, a["B"], a["base"], ex["seq_lens"], ex["req_slots"],
                       ex["lora_ranks"], ex["scalings"], ex["slice_offsets"])
        e = mod.embedding_a(ex["input_ids"], a["A_emb"], ex["seq_lens"], ex["req_slots"],
                            ex["lora_ranks"], ex["vocab_size"])
        if not (np.array_equal(h, a["h"]) and np.array_equal(y, a["y"])
                and np.array_equal(e, a["e"])):
            return False
        rng = np.random.default_rng(11)
        for _ in range(5):
            case = _random_case(rng)
            want = _brute(case)
            c, R = case["c"], case["R"]
            for slot, rho in enumerate(case["ranks"]):
                for k in range(c):
                    case["A"][slot, k * R + rho:(k + 1) * R, :] = np.nan
                case["B"][slot, :, rho:] = np.nan
            got = mod.lora_forward(case["x"], case["A"], case["B"], case["base"],
                                   case["lens"], case["slots"], case["ranks"],
                                   case["scal"], case["offs"])
            if not np.allclose(got, want, rtol=1e-12, atol=1e-12):
                return False
    except Exception:
        return False
    return True


def test_pins_pass_on_oracle():
    assert _pins_pass(ol)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    assert not _pins_pass(_mutant_module(MUTANTS[name])), name


# ------------------------------------------------------------- lm_head plans

def test_lm_head_plan_hand_example():
    ex = json.load(open(os.path.join(GOLDEN, "lm_head_plan_example.json")))
    got = op.lm_head_plan(ex["pruned_lens"], ex["req_slots"], 128, ex["chunk_size_override"])
    for k, v in ex["expected"].items():
        assert got[k] == v, k


def test_lm_head_segments_are_runs_of_the_original_order():
    """Brute force over tiny batches: merging consecutive same-slot requests
    and chunking the runs equals cutting the runs of equal slots of the
    token sequence in ORIGINAL order (no sort) into chunks -- the plan's
    segment rule applied to the unsorted slot sequence."""
    for bs in range(0, 5):
        for lens in itertools.product(range(0, 4), repeat=bs):
            for slots in itertools.product(range(0, 3), repeat=bs):
                for chunk in (1, 2, 3, 16):
                    seg_slots, seg_lens = op.merge_and_chunk(list(slots), list(lens), chunk)
                    want_slots, want_indptr = op.segments(op.token_slots(lens, slots), chunk)
                    assert seg_slots == want_slots
                    got_indptr = [0]
                    for n in seg_lens:
                        got_indptr.append(got_indptr[-1] + n)
                    assert got_indptr == want_indptr


def test_lm_head_plan_invariants_and_chunk_rule():
    rng = random.Random(7)
    for _ in range(200):
        bs = rng.randint(1, 40)
        lens = [rng.choice([0, 1, 1, 1, 2, 5, 40, 300]) for _ in range(bs)]
        slots = [rng.randrange(4) for _ in range(bs)]
        for cap in (16, 64, 128):
            pl = op.lm_head_plan(lens, slots, cap)
            total = sum(lens)
            assert pl["chunk_size"] == op.chunk_size_for_tokens(total, cap)
            assert pl["permutation"] == list(range(total))
            ind = pl["seg_indptr"]
            assert ind[0] == 0 and ind[-1] == total
            assert all(0 < ind[i + 1] - ind[i] <= pl["chunk_size"] for i in range(pl["num_segments"]))
            # tokens of a segment all belong to requests of the segment's slot
            rows = op.token_slots(lens, slots)
            for i in range(pl["num_segments"]):
                assert set(rows[ind[i]:ind[i + 1]]) == {pl["seg_slots"][i]}
            # a segment is followed by one of its own slot only when it is a full chunk
            for i in range(pl["num_segments"] - 1):
                if pl["seg_slots"][i] == pl["seg_slots"][i + 1]:
                    assert ind[i + 1] - ind[i] == pl["chunk_size"]
    padded = op.lm_head_plan([3, 0, 4], [1, 0, 1], 128, capacity=5)
    assert padded["seg_slots"] == [1, 0, 0, 0, 0]
    assert padded["seg_indptr"] == [0, 7, 7, 7, 7, 7]



# ------------------------------------------ planted mistakes in the planner

def _plan_pins_pass(mod):
    """Run the page's worked examples, the hand-derived plans and the chunk
    table against a planner module (expected values written by hand)."""
    try:
        ex = _load("plan_worked_examples.json")
        pe, se, tiny = ex["permutation_example"], ex["segments_example"], ex["tiny_plan_hand_derived"]
        p = mod.plan(pe["seq_lens"], pe["seq_weight_indices"], False, 128,
                     chunk_override=se["chunk_size"])
        if (p["permutation"], p["seg_slots"], p["seg_indptr"]) != (
                pe["permutation"], se["weight_indices"], se["seg_indptr"]):
            return False
        p = mod.plan(tiny["seq_lens"], tiny["req_slots"], tiny["is_decode"], tiny["max_chunk_size"])
        if any(p[k] != tiny[k] for k in ("chunk_size", "permutation", "seg_indptr", "seg_slots",
                                         "req_seg_indptr")):
            return False
        for cap, row in CHUNK_TABLE.items():
            if [mod.chunk_size_for_tokens(n, cap) for n in CHUNK_TABLE_TOKENS] != row:
                return False
        # graph padding: slot 0, zero-length segments (worked by hand)
        p = mod.plan([2, 1, 3], [1, 0, 1], False, 128, capacity=5)
        if (p["permutation"], p["seg_slots"], p["seg_indptr"]) != (
                [2, 0, 1, 3, 4, 5], [0, 1, 0, 0, 0], [0, 1, 6, 6, 6, 6]):
            return False
        lm = _load("lm_head_plan_example.json")
        got = mod.lm_head_plan(lm["pruned_lens"], lm["req_slots"], 128, lm["chunk_size_override"])
        if any(got[k] != v for k, v in lm["expected"].items()):
            return False
        # a zero-token request of another slot does not split a run
        got = mod.lm_head_plan([3, 0, 4], [1, 0, 1], 128)
        if (got["seg_slots"], got["seg_indptr"]) != ([1], [0, 7]):
            return False
        # the chunk follows the pruned token count (300 tokens -> 128), not the request count
        got = mod.lm_head_plan([300], [0], 128)
        if (got["chunk_size"], got["seg_indptr"]) != (128, [0, 128, 256, 300]):
            return False
    except Exception:
        return False
    return True


PLAN_MUTANTS = {
    "sort descending": [
        ("pairs = sorted((slot, t) for t, slot in enumerate(rows))",
         "pairs = sorted(((slot, t) for t, slot in enumerate(rows)), reverse=True)")],
    "ties in reverse token order": [
        ("pairs = sorted((slot, t) for t, slot in enumerate(rows))",
         "pairs = [(a, -b) for a, b in sorted((slot, -t) for t, slot in enumerate(rows))]")],
    "remainder first": [
        ("seg_lens.append(chunk if q < pieces - 1 else run - (pieces - 1) * chunk)",
         "seg_lens.append(run - (pieces - 1) * chunk if q == 0 else chunk)")],
    "256 threshold exclusive": [("if num_tokens >= 256:", "if num_tokens > 256:")],
    "server cap ignored": [("return min(max_chunk_size, wanted)", "return wanted")],
    "graph padding repeats the last slot": [
        ("seg_slots = seg_slots + [0] * (capacity - num_segments)",
         "seg_slots = seg_slots + seg_slots[-1:] * (capacity - num_segments)")],
    "request boundaries count requests": [
        ("out.append(out[-1] + length)", "out.append(out[-1] + 1)")],
    "lm_head runs not merged": [("if runs and runs[-1][0] == slot:", "if False:")],
    "lm_head zero-token requests kept": [
        ("        if n == 0:\n            continue\n", "")],
    "lm_head remainder first": [
        ("seg_lens.append(chunk if q < pieces - 1 else n - (pieces - 1) * chunk)",
         "seg_lens.append(n - (pieces - 1) * chunk if q == 0 else chunk)")],
    "lm_head chunk from request count": [
        ("chunk_size_for_tokens(total, max_chunk_size)",
         "chunk_size_for_tokens(len(pruned_lens), max_chunk_size)")],
    "lm_head tokens sorted by slot": [
        ('"permutation": list(range(total)),',
         '"permutation": gather_permutation(token_slots(pruned_lens, req_slots))[0],')],
}


def _plan_mutant_module(edits):
    import types
    src = open(op.__file__).read()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new, 1)
    mod = types.ModuleType("plan_mutant")
    exec(compile(src, "plan_mutant", "exec"), mod.__dict__)
    return mod


def test_plan_pins_pass_on_oracle():
    assert _plan_pins_pass(op)


@pytest.mark.parametrize("name", sorted(PLAN_MUTANTS))
def test_plan_pins_catch_planted_mistake(name):
    assert not _plan_pins_pass(_plan_mutant_module(PLAN_MUTANTS[name])), name
