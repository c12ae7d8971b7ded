"""Host checks of the benchmark's contract (no GPU): the one-GPU refusal and
the algorithmic byte counts its roofline figures divide by.

The byte counts are recomputed here from the workload shapes by hand
(row bytes, probe rows skipped, rank-state and mean reads), independently
of bench.py's own bookkeeping.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synthetic import CONFIGS  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _apply_bytes(c):
    """One plane's apply: every non-probe row read and written, its rank-state
    row read; the rank factor B and the mean once per unit; weights and probe
    bits once per segment."""
    units = c.n_layers * c.n_segs * c.n_kv_heads
    row = 2 * c.head_dim                                  # bf16
    rows = units * (c.n_tokens - c.b)
    state = units * c.rank * c.head_dim * 4
    weights = c.n_segs * c.n_tokens * 4 if c.weight == "clip" else 0
    bits = c.n_segs * ((c.n_tokens + 31) // 32) * 4
    return rows * (2 * row + 4 * c.rank) + state + units * c.head_dim * 4 + weights + bits


@pytest.mark.parametrize("name,expected", [
    ("c2", 471_192_064),          # the per-launch figures the profiles quote
    ("c4", 5_798_367_232),
    ("c5", 39_285_899_264),
])
def test_roofline_bytes_per_launch(name, expected):
    c = CONFIGS[name]
    assert _apply_bytes(c) == expected
    w = bench.Workload.ALL[name](c, None, None)
    assert w.alg_bytes()["roofline_per_launch"] == expected
