"""The host code of libsgg_lora under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only).

tests/native/sanitize_driver.cpp is linked with the planner (plan.cpp), the
shrink tile choice (tiling.cpp) and the C-ABI entry points (lora_api.hip),
all built with host-side -fsanitize=address,undefined; the kernel launchers
are stubs.  The driver plans every batch it is sent into exactly-sized heap
buffers, so an out-of-bounds read or write, or undefined behaviour, stops it
with a sanitizer report.  Its plans are compared with the oracle bit for bit,
and its validation cases must return the documented status codes.
"""

import itertools
import os
import random
import shutil
import subprocess

import numpy as np
import pytest

from oracle import plan as op
from synth import CONFIGS, draw_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "segmented_gather_gemm_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "native", "sanitize_driver.cpp")
REGIONS = 10
WORK_TOKENS = 128


def _hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("asan") / "sanitize_driver")
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           DRIVER, os.path.join(CSRC, "lora_api.hip"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "tiling.cpp"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


def _run(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         env=env, timeout=600)
    report = res.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert res.returncode == 0, report[-4000:]
    return res.stdout.splitlines()


def _fields(line):
    parts = line.split("|")
    return [int(v) for v in parts[0].split()], [[int(v) for v in p.split()] for p in parts[1:]]


def _plan_cmd(lens, slots, L, decode, max_chunk, override, cap):
    has = 0 if lens is None else 1
    vals = ([] if lens is None else list(lens)) + list(slots)
    return " ".join(map(str, ["P", int(decode), max_chunk, override, L, cap, has, len(slots)]
                        + vals))


def _check_plan(out, lens, slots, L, decode, max_chunk, override, cap):
    head, arrays = _fields(out)
    ref = op.plan(lens, slots, decode, max_chunk, override, capacity=cap)
    assert head[0] == 0, (lens, slots, head)
    assert head[1:] == [ref["num_segments"], ref["chunk_size"], ref["num_tokens"]]
    perm, ind, sl, req = arrays
    assert perm == ref["permutation"]
    assert ind == ref["seg_indptr"] and sl == ref["seg_slots"]
    assert req == ref["req_seg_indptr"]


def _capacity(s, L, override):
    min_chunk = override if override > 0 else 16
    if s <= 0:
        return 0
    return min(s, -(-s // min_chunk) + L)


def test_planner_exhaustive_and_random_under_sanitizers(driver):
    cases = []
    for bs in range(0, 4):
        for lens in itertools.product(range(4), repeat=bs):
            for slots in itertools.product(range(3), repeat=bs):
                for override in (1, 2, 3, 0):
                    cases.append((list(lens), list(slots), 3, False, 128, override))
    rng = random.Random(7)
    for _ in range(400):
        bs = rng.randint(0, 80)
        L = rng.randint(1, 16)
        lens = [rng.choice([0, 1, 1, 2, 3, 15, 16, 17, 100, 300]) for _ in range(bs)]
        slots = [rng.randrange(L) for _ in range(bs)]
        cases.append((lens, slots, L, False, rng.choice([1, 8, 16, 17, 32, 48, 64, 128, 256]),
                      rng.choice([0, 0, 0, 1, 5, 16])))
    for _ in range(100):
        bs = rng.randint(0, 300)
        L = rng.randint(1, 40)
        cases.append((None, [rng.randrange(L) for _ in range(bs)], L, True,
                      rng.choice([16, 64, 128]), 0))
    lines, caps = [], []
    for lens, slots, L, decode, mc, ov in cases:
        s = len(slots) if lens is None else sum(lens)
        cap = _capacity(s, L, ov) + rng.choice([0, 0, 3])   # some with padding
        caps.append(cap)
        lines.append(_plan_cmd(lens, slots, L, decode, mc, ov, cap))
    out = _run(driver, lines)
    assert len(out) == len(cases)
    for line, (lens, slots, L, decode, mc, ov), cap in zip(out, cases, caps):
        _check_plan(line, lens, slots, L, decode, mc, ov, cap)


def test_planner_rejects_under_sanitizers(driver):
    lines = [
        "P 0 128 0 4 8 1 2 1 2 0 5",       # slot 5 >= max_loras 4
        "P 0 128 0 4 8 1 2 1 -2 0 1",      # negative length
        "P 1 128 0 4 8 1 2 1 2 0 1",       # decode with a 2-token request
        "P 0 128 0 4 0 1 2 30 30 0 1",     # capacity 0 for 4 segments
        "P 0 128 -1 4 8 1 1 3 0",          # negative override
    ]
    out = _run(driver, lines)
    codes = [int(line.split()[0]) for line in out]
    assert codes == [-3, -1, -1, -3, -1]


def test_lm_head_planner_under_sanitizers(driver):
    cases = []
    for bs in range(0, 4):
        for lens in itertools.product(range(3), repeat=bs):
            for slots in itertools.product(range(3), repeat=bs):
                cases.append((list(lens), list(slots), 0))
    rng = random.Random(11)
    for _ in range(200):
        bs = rng.randint(0, 60)
        cases.append(([rng.choice([0, 1, 1, 2, 5, 40]) for _ in range(bs)],
                      [rng.randrange(5) for _ in range(bs)], rng.choice([0, 0, 3])))
    lines, caps = [], []
    for lens, slots, ov in cases:
        s = sum(lens)
        cap = _capacity(s, max(len(slots), 1), ov)
        caps.append(cap)
        lines.append(" ".join(map(str, ["H", 128, ov, 5, cap, len(slots)] + lens + slots)))
    out = _run(driver, lines)
    for line, (lens, slots, ov), cap in zip(out, cases, caps):
        head, arrays = _fields(line)
        ref = op.lm_head_plan(lens, slots, 128, ov, capacity=cap)
        assert head[0] == 0
        assert head[1:] == [ref["num_segments"], ref["chunk_size"], ref["num_tokens"]]
        assert arrays[0] == ref["permutation"]
        assert arrays[1] == ref["seg_indptr"] and arrays[2] == ref["seg_slots"]


def _layout(tok_cap, seg_cap, req_cap, L):
    sizes = [tok_cap, seg_cap + 1, seg_cap, req_cap + 1, req_cap, L, L, seg_cap + 1, seg_cap,
             tok_cap]
    offs, pos = [], 0
    for n in sizes:
        offs.append(pos)
        pos += -(-n // 64) * 64
    return offs, sizes


def _upload_cmd(lm_head, lens, slots, ranks, scal, L, decode, mc, tok_cap, seg_cap, req_cap):
    bits = np.asarray(scal, np.float32).view(np.int32).tolist()
    has = 0 if lens is None else 1
    vals = ([] if lens is None else list(lens)) + list(slots) + list(ranks) + bits
    return " ".join(map(str, ["U", int(lm_head), int(decode), mc, 0, L, tok_cap, seg_cap,
                              req_cap, has, len(slots)] + vals))


def test_plan_upload_staging_under_sanitizers(driver):
    """lora_plan_upload / lora_plan_lm_head_upload plan into an exactly-sized
    staging buffer: every region equals the oracle plan and the tables, and
    the work segments partition the same sorted positions (the transfer is a
    stub)."""
    cases = []
    for name in CONFIGS:
        b = draw_batch(name)
        lens = None if b.is_decode else list(b.seq_lens)
        s = b.num_tokens
        cap = _capacity(s, b.num_loras, 0)
        cases.append((False, lens, b, s, cap, len(b.req_slots)))
        cases.append((False, lens, b, s + 37, cap + 5, len(b.req_slots) + 2))  # graph padding
    b = draw_batch("decode")
    cases.append((True, [1] * len(b.req_slots), b, b.num_tokens, b.num_tokens, len(b.req_slots)))
    lines = [_upload_cmd(lm, lens, b.req_slots, b.lora_ranks, b.scalings, b.num_loras,
                         b.is_decode and not lm, b.max_chunk_size, tc, sc, rc)
             for lm, lens, b, tc, sc, rc in cases]
    out = _run(driver, lines)
    for line, (lm, lens, b, tok_cap, seg_cap, req_cap) in zip(out, cases):
        head, arrays = _fields(line)
        info, staging = arrays
        assert head[0] == 0, head
        offs, sizes = _layout(tok_cap, seg_cap, req_cap, b.num_loras)
        reg = [staging[o:o + n] for o, n in zip(offs, sizes)]
        if lm:
            ref = op.lm_head_plan(lens, b.req_slots, b.max_chunk_size, capacity=seg_cap)
        else:
            ref = op.plan(lens, b.req_slots, b.is_decode, b.max_chunk_size, capacity=seg_cap)
        s = ref["num_tokens"]
        assert info[:2] == [ref["num_segments"], ref["chunk_size"]]
        assert reg[0][:s] == ref["permutation"]
        assert reg[1] == ref["seg_indptr"] and reg[2] == ref["seg_slots"]
        assert reg[4][:len(b.req_slots)] == list(b.req_slots)
        assert reg[5] == list(b.lora_ranks)
        assert np.array_equal(np.asarray(reg[6], np.int32).view(np.float32),
                              np.asarray(b.scalings, np.float32))
        # work segments: merged runs of one slot over the sorted tokens
        n_work = info[4]
        wind, wsl = reg[7][:n_work + 1], reg[8][:n_work]
        assert wind[0] == 0 and wind[-1] == s
        assert all(wind[i] < wind[i + 1] for i in range(n_work))
        limit = max(ref["chunk_size"], WORK_TOKENS)
        assert all(wind[i + 1] - wind[i] <= limit for i in range(n_work))
        sorted_slots = np.sort(np.repeat(np.asarray(b.req_slots), lens or 1), kind="stable")
        for w in range(n_work):
            assert set(sorted_slots[wind[w]:wind[w + 1]].tolist()) == {wsl[w]}
        assert reg[7][n_work + 1:] == [s] * (seg_cap - n_work)   # padding: empty, slot 0
        assert reg[8][n_work:] == [0] * (seg_cap - n_work)


def test_plan_upload_embedding_under_sanitizers(driver):
    """lora_plan_upload_embedding writes the same staging buffer and plan
    info as lora_plan_upload, and takes the one-launch form exactly for
    decode-shaped batches of at most 3072 tokens over at most 64 slots,
    handing that launch each token's slot and the slots' ranks clamped to
    [0, R]."""
    rng = random.Random(5)
    cases = []   # (lens or None, slots, ranks, L, decode, R, fused)
    for bs, L, decode, fused in [(256, 8, True, True), (3072, 64, True, True),
                                 (3073, 8, True, False), (100, 65, True, False),
                                 (1, 1, True, True), (0, 4, True, False)]:
        cases.append((None, [rng.randrange(L) for _ in range(bs)],
                      [rng.choice([-3, 0, 4, 16, 40]) for _ in range(L)], L, decode, 16, fused))
    cases.append(([1] * 50, [rng.randrange(5) for _ in range(50)], [16, 0, 8, 20, 3], 5, False,
                  16, True))
    cases.append(([1, 2, 1], [0, 1, 0], [16, 8], 2, False, 16, False))
    # (token, j) pairs past 2^31: the two launches (the fused launch indexes them in int32)
    cases.append((None, [rng.randrange(8) for _ in range(3072)], [16] * 8, 8, True, 1 << 20,
                  False))
    cases.append((None, [rng.randrange(8) for _ in range(2048)], [16] * 8, 8, True, 1 << 19,
                  True))
    cases.append(([1, 0, 1], [0, 1, 0], [16, 8], 2, False, 16, False))
    lines = []
    for lens, slots, ranks, L, decode, R, _ in cases:
        s = len(slots) if lens is None else sum(lens)
        cap = max(_capacity(s, L, 0), 1)
        scal = [1.0 + 0.25 * a for a in range(L)]
        u = _upload_cmd(False, lens, slots, ranks, scal, L, decode, 128, s, cap, len(slots))
        lines.append(u)
        lines.append(" ".join(["E"] + u.split()[2:3] + u.split()[3:4] + u.split()[5:]
                              + [str(R)]))
    out = _run(driver, lines)
    assert len(out) == 2 * len(cases)
    for (lens, slots, ranks, L, decode, R, fused), u, e in zip(cases, out[0::2], out[1::2]):
        uhead, (uinfo, ustaging) = _fields(u)
        parts = e.split("|")
        assert int(parts[0].split()[0]) == 0 and uhead[0] == 0, (e[:200], u[:200])
        assert [int(v) for v in parts[1].split()] == uinfo
        assert [int(v) for v in parts[2].split()] == ustaging
        flag, s_k, R_k, n_k = [int(v) for v in parts[3].split()]
        assert flag == int(fused), (len(slots), L, lens)
        if fused:
            s = len(slots)
            offs, _ = _layout(s, max(_capacity(s, L, 0), 1), len(slots), L)
            assert (s_k, R_k, n_k) == (s, R, offs[9])
            assert [int(v) for v in parts[4].split()] == list(slots)
            want = [min(max(r, 0), R) for r in ranks] + [0] * (64 - L)
            assert [int(v) for v in parts[5].split()] == want


EXPECTED = {
    "shrink_ok": 0, "shrink_null_x": -1, "shrink_k0": -1, "shrink_c9": -1, "shrink_k_odd": -2,
    "shrink_ldh_small": -1, "shrink_misaligned": -2, "shrink_empty_plan": 0,
    "expand_ok": 0, "expand_stacked_ok": 0, "expand_offsets_decrease": -1,
    "expand_max_slice_small": -1, "expand_rank_above_128": -2, "expand_b_rows_short": -1,
    "expand_null_base": -1, "qkv_ok": 0, "qkv_workspace_small": -3, "workspace_sizes": 0,
    "embedding_ok": 0, "embedding_extra_vocab": -2, "embedding_vocab_above_v": -1,
    "plan_device_ok": 0, "plan_device_too_many_loras": -2, "plan_device_buffer_small": -3,
    "moe_plan_ok": 0, "moe_plan_too_many_copies": -2, "moe_plan_too_many_virtual": -2,
    "moe_plan_buffer_small": -3, "moe_plan_null_plan": -1,
}


def test_entry_point_validation_under_sanitizers(driver):
    out = _run(driver, ["V"])
    assert out[-1] == "end"
    got = dict(line.split() for line in out[:-1])
    launches = int(got.pop("launches"))
    assert {k: int(v) for k, v in got.items()} == EXPECTED
    assert launches >= 6   # the accepted calls reached their (stub) launchers
