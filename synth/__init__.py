"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This package draws batch structure (sequence lengths, adapter assignment,
ranks, scalings) and tensor values from fixed NumPy PCG64 seeds.  It holds no
part of the LoRA arithmetic or of the planner: both the HIP path and the
oracle consume what it returns.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    Batch,
    Projection,
    draw_batch,
    draw_embedding,
    draw_ids,
    draw_projection,
    to_f64,
)
