"""Pins for the MoE LoRA oracle (oracle/moe.py): checked against things other
than itself -- a hand example (tests/golden/moe_lora_hand_example.json), the
reduction to the dense LoRA oracle with one expert and top-1 routing, an
invariance under request order, rank padding filled with NaN, and planted
mistakes that these pins must catch."""

import json
import os
import types

import numpy as np
import pytest

from oracle import lora as ol
from oracle import moe as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand():
    with open(os.path.join(GOLDEN, "moe_lora_hand_example.json")) as f:
        ex = json.load(f)
    return ex, {k: np.asarray(ex[k], dtype=np.float64)
                for k in ("x", "A", "B", "out_before", "out_after")}


def _random_case(rng, bs=5, L=3, E=4, k=2, R=4, K=6, N=5):
    lens = [int(v) for v in rng.integers(0, 4, size=bs)]
    slots = [int(v) for v in rng.integers(0, L, size=bs)]
    s = sum(lens)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ranks = [int(v) for v in rng.integers(0, R + 1, size=L)]
    return {"indptr": indptr, "slots": slots, "ranks": ranks,
            "scal": [float(v) for v in rng.uniform(-2, 2, size=L)],
            "topk": rng.integers(0, E, size=(s, k)), "E": E, "k": k, "lens": lens,
            "x": rng.standard_normal((s, K)), "A": rng.standard_normal((L, E, R, K)),
            "B": rng.standard_normal((L, E, N, R)), "out": rng.standard_normal((s * k, N))}


def test_hand_example():
    ex, a = _hand()
    v = om.virtual_experts(ex["req_seg_indptr"], ex["req_weight_indices"], ex["topk_ids"],
                           ex["num_experts"])
    assert v.tolist() == ex["virtual_experts"]
    y = om.moe_lora_add(a["x"], a["A"], a["B"], a["out_before"], ex["req_seg_indptr"],
                        ex["req_weight_indices"], ex["topk_ids"], ex["lora_ranks"],
                        ex["scalings"])
    np.testing.assert_array_equal(y, a["out_after"])


def test_one_expert_top1_is_the_dense_lora_forward():
    """With E = 1 and k = 1 every copy is its token and every virtual expert
    its adapter: the add is the plain LoRA shrink + expand of the dense
    oracle (itself pinned in test_oracle.py), with the request lengths that
    req_seg_indptr encodes."""
    rng = np.random.default_rng(3)
    for _ in range(6):
        c = _random_case(rng, E=1, k=1)
        got = om.moe_lora_add(c["x"], c["A"], c["B"], c["out"], c["indptr"], c["slots"],
                              c["topk"], c["ranks"], c["scal"])
        N = c["B"].shape[2]
        want = ol.lora_forward(c["x"], c["A"][:, 0], c["B"][:, 0], c["out"], c["lens"],
                               c["slots"], c["ranks"], c["scal"], [0, N])
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_request_order_invariance():
    """Reordering the requests (their tokens, routing rows and output rows
    move with them) reorders the result the same way."""
    rng = np.random.default_rng(5)
    for _ in range(4):
        c = _random_case(rng)
        y = om.moe_lora_add(c["x"], c["A"], c["B"], c["out"], c["indptr"], c["slots"],
                            c["topk"], c["ranks"], c["scal"])
        order = rng.permutation(len(c["lens"]))
        k = c["k"]
        tok = np.concatenate([np.arange(c["indptr"][r], c["indptr"][r + 1]) for r in order]
                             + [np.zeros(0, np.int64)]).astype(np.int64)
        rows = (tok[:, None] * k + np.arange(k)[None, :]).reshape(-1)
        lens2 = [c["lens"][r] for r in order]
        indptr2 = np.concatenate([[0], np.cumsum(lens2)]).astype(np.int64)
        y2 = om.moe_lora_add(c["x"][tok], c["A"], c["B"], c["out"][rows], indptr2,
                             [c["slots"][r] for r in order], c["topk"][tok], c["ranks"],
                             c["scal"])
        np.testing.assert_allclose(y2, y[rows], rtol=1e-12, atol=1e-12)


def test_rank_padding_is_never_read():
    """A and B entries past an adapter's rank set to NaN change nothing."""
    rng = np.random.default_rng(7)
    for _ in range(4):
        c = _random_case(rng)
        y = om.moe_lora_add(c["x"], c["A"], c["B"], c["out"], c["indptr"], c["slots"],
                            c["topk"], c["ranks"], c["scal"])
        A, B = c["A"].copy(), c["B"].copy()
        for a, rho in enumerate(c["ranks"]):
            A[a, :, rho:, :] = np.nan
            B[a, :, :, rho:] = np.nan
        y2 = om.moe_lora_add(c["x"], A, B, c["out"], c["indptr"], c["slots"], c["topk"],
                             c["ranks"], c["scal"])
        np.testing.assert_array_equal(y2, y)


# ------------------------------------------------------- planted mistakes

MUTANTS = {
    "copy row j * s + t": [("y[t * k + j] +=", "y[j * s + t] +=")],
    "expert of copy 0 for every copy": [("e = int(topk_ids[t, j])", "e = int(topk_ids[t, 0])")],
    "adapter of the token index as a request": [
        ("a = int(req_weight_indices[req[t]])\n        rho",
         "a = int(req_weight_indices[min(t, len(req_weight_indices) - 1)])\n        rho")],
    "scaling dropped": [("y[t * k + j] += sigma * (B", "y[t * k + j] += (B")],
    "virtual expert e * L + a": [
        ("v[t * k + j] = a * num_experts + int(topk_ids[t, j])",
         "v[t * k + j] = int(topk_ids[t, j]) * len(req_weight_indices) + a")],
    "request ranges shifted by one token": [
        ("for t in range(int(req_seg_indptr[r]), int(req_seg_indptr[r + 1])):",
         "for t in range(int(req_seg_indptr[r]) + 1, int(req_seg_indptr[r + 1]) + 1):\n"
         "            if t >= num_tokens:\n                break")],
    "rank padding read": [("h = A[a, e, :rho, :] @ x[t]", "h = A[a, e, :, :] @ x[t]"),
                          ("(B[a, e, :, :rho] @ h)", "(B[a, e, :, :] @ h)")],
}


def _mutant(edits):
    src = open(om.__file__).read()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new, 1)
    mod = types.ModuleType("moe_mutant")
    exec(compile(src, "moe_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    try:
        ex, a = _hand()
        v = mod.virtual_experts(ex["req_seg_indptr"], ex["req_weight_indices"],
                                ex["topk_ids"], ex["num_experts"])
        y = mod.moe_lora_add(a["x"], a["A"], a["B"], a["out_before"], ex["req_seg_indptr"],
                             ex["req_weight_indices"], ex["topk_ids"], ex["lora_ranks"],
                             ex["scalings"])
        if v.tolist() != ex["virtual_experts"] or not np.array_equal(y, a["out_after"]):
            return False
        rng = np.random.default_rng(9)
        for _ in range(4):
            c = _random_case(rng)
            y = mod.moe_lora_add(c["x"], c["A"], c["B"], c["out"], c["indptr"], c["slots"],
                                 c["topk"], c["ranks"], c["scal"])
            A, B = c["A"].copy(), c["B"].copy()
            for ad, rho in enumerate(c["ranks"]):
                A[ad, :, rho:, :] = np.nan
                B[ad, :, :, rho:] = np.nan
            y2 = mod.moe_lora_add(c["x"], A, B, c["out"], c["indptr"], c["slots"], c["topk"],
                                  c["ranks"], c["scal"])
            if not np.array_equal(y, y2):
                return False
    except Exception:
        return False
    return True


def test_pins_pass_on_oracle():
    assert _pins_pass(om)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    assert not _pins_pass(_mutant(MUTANTS[name])), name
