"""Seeded synthetic inputs for the KV-correction path (shapes + random draws only).

This package holds the five workload shapes and the seeded random draws that
build their inputs.  It contains none of the correction method's arithmetic:
no rotary rotation, no scoring, no selection, no mean fit, no diff coding.
Both the oracle tests and the GPU benchmark draw their inputs from here.
"""
from .workloads import (  # noqa: F401
    CONFIGS,
    WorkloadConfig,
    draw_anchor_pool,
    draw_correction,
    draw_collective,
    draw_draft_queries,
    draw_page_table,
    draw_deltas,
    make_gen,
)
