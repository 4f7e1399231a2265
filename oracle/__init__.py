"""Reference oracle for chunked SGMV LoRA: test infrastructure, not product code.

This package is a plain, slow and deliberately obvious CPU implementation of
what the chunked SGMV LoRA path computes.  It exists so that the HIP path can
be checked against something written independently from it:

* ``oracle.plan``   -- the batch planner (chunk-size rule, gather permutation,
  segmenting, per-request routing), pure Python over lists, bit-exact integers.
* ``oracle.lora``   -- the per-token mathematics (LoRA-A shrink, LoRA-B expand
  with scaling and stacked slice offsets, LoRA-A embedding gather) in float64
  NumPy, computed from the *requests*, never from a plan.
* ``oracle.moe``    -- per-request routing to MoE "virtual experts" (adapter x
  expert) and the LoRA add on a fused-MoE intermediate, in float64, from the
  per-request fields req_seg_indptr / req_weight_indices (PR #24007 report
  page); the kernel body is not on the pages, so the reading used is stated
  in that module.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The library under
``segmented_gather_gemm_amd`` never imports it, and this package imports
nothing from that library: the two share no code.

Sources are the web pages on sglang's chunked LoRA backend: the
``chunked_backend.py`` page (class ``ChunkedSgmvLoRABackend``), the
``base_backend.py`` page (class ``BaseLoRABackend`` and its shape
contracts), the ``lora_manager.py`` page (per-slot rank and scaling
tables) and the PR #24007 report page (per-request routing for MoE).  Each
function names the passage it follows.

Parity status: every function here is pinned by tests in
``tests/test_oracle.py`` and ``tests/test_oracle_moe.py`` against values
printed on the pages or worked by hand, closed forms, brute force,
reductions to other pinned functions and invariants; none is "parity
unpinned".
"""

from . import lora, moe, plan  # noqa: F401
