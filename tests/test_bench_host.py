"""bench.py's byte accounting on the host (no GPU): the algorithmic bytes per parameter that
the roofline and the step GB/s are computed from.

A step with k micro-batches reads and writes 10k + 24 bytes per parameter when the last
micro-batch is folded into the norm and AdamW passes (k >= 2): 6 for the first
accumulation, 10 for each further one, 6 for the norm (fp32 accumulator + 16-bit last
gradient) and 32 for AdamW (18 read, 14 written).  With one micro-batch there is no
accumulator: the norm reads the 16-bit gradient (2) and AdamW 28 bytes, 30 in all.  The
model state itself is 16 bytes per parameter ('Chapter 41 Training at Scale', equation 41.1)
plus the 4-byte accumulator.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_step_bytes_follow_the_schedule():
    for k in (2, 3, 4, 8, 16):
        b = bench.bytes_per_param(k)
        assert b["step"] == 10 * k + 24
        assert b["step"] == b["accumulate_first"] + (k - 2) * b["accumulate"] + b["norm"] + b["adamw"]
        assert b["adamw"] == 32 and b["norm"] == 6
    b1 = bench.bytes_per_param(1)
    assert b1["step"] == 30 and b1["norm"] + b1["adamw"] == 30 and b1["adamw"] == 28


def test_group_bytes_reduce_to_the_one_at_a_time_schedule():
    """Groups of one micro-batch give the one-at-a-time step's 10k + 24 bytes, and k = 1 its 30;
    folding resident micro-batches saves the accumulator's round trips: for k = 4, 50 bytes with
    two accumulated in one pass, and 42 with all four folded into the norm and AdamW."""
    for k in (2, 3, 4, 8):
        ones = [[i] for i in range(k - 1)]
        assert bench.group_bytes_per_param(ones, [k - 1]) == bench.bytes_per_param(k)["step"]
    assert bench.group_bytes_per_param([], [0]) == bench.bytes_per_param(1)["step"] == 30
    assert bench.group_bytes_per_param([[0, 1]], [2, 3]) == 8 + 8 + 34 == 50
    assert bench.group_bytes_per_param([], [0, 1, 2, 3]) == 8 + 34 == 42
    assert bench.group_bytes_per_param([[0, 1, 2, 3]], [4, 5, 6, 7]) == 12 + 12 + 38 == 62


def test_adamw_bytes_are_the_state_it_touches():
    """AdamW reads acc (4), the last 16-bit gradient (2), master, m, v (12) and writes master, m,
    v (12) and the 16-bit weight (2): every byte of the 20-byte state except the gradient buffers
    of the other micro-batches, once."""
    b = bench.bytes_per_param(4)
    read = 4 + 2 + 4 + 4 + 4
    written = 4 + 4 + 4 + 2
    assert b["adamw"] == read + written == 32


def test_more_than_one_gpu_is_refused_without_touching_a_gpu():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and r.stdout == ""


def test_unknown_extras_are_refused_before_any_work():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--extras",
                        "resident_groups,nonsense"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and r.stdout == "" and "nonsense" in r.stderr


def test_launches_per_step_match_the_traced_steps():
    """The launches bench.py reports per step, against the kernels the traces of its steps show
    (profiles/kernel_trace_*.md): the k - 1 accumulations (the token weights inside the first,
    their own launch when k = 1), the norm's first stage, its second stage above 8192 partial
    sums, its finish, AdamW, and the clock and the scaler unless one call folds them into the
    finish."""
    cases = [  # (k, chunks, eager launches, captured launches)
        (4, 5153, 8, 6),          # llama-10.5M
        (1, 60842, 6, 4),         # gpt-124M: one 16-bit stream, 16 chunks per norm block
        (8, 642490, 13, 11),      # gpt-1.3B
        (4, 328215, 9, 7),        # ragged-4096
        (4, 3921026, 9, 7),       # llama3-8B
    ]
    for k, chunks, eager, captured in cases:
        assert bench.launches_per_step(k, chunks, False) == eager, (k, chunks)
        assert bench.launches_per_step(k, chunks, True) == captured, (k, chunks)
