"""Parity at the full sizes the benchmark times (needs an MI355X with ~210 GB free).

The device runs the whole tensor list in the launch configuration and memory layout
bench.py uses (flattened buffers, per-tensor views);
the oracle recomputes the global norm from regenerated inputs every step
(streamed, all elements) and the update on sampled windows: the first and last
512 elements of every tensor plus 64 seeded random windows of 4099 elements.
"""
import pytest

from inputs import configs

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.timeout(1100)
@pytest.mark.parametrize("name,steps", [("ragged-4096", 2), ("llama3-8B", 2), ("huge-tensor", 2)])
def test_full_size_sampled_parity(name, steps, progress):
    """The 8B list runs bench.py's eager step exactly: the token weights computed from device
    counts inside the first accumulation, every pass reading its weight on the device, the
    norm, AdamW and scaler as three calls.  The other lists run the host-weight calls."""
    run_sampled_parity(name, steps, say=progress, bench_sequence=name == "llama3-8B")


@pytest.mark.timeout(1100)
@pytest.mark.parametrize("name,schedule", [
    ("llama3-8B", ([], [0, 1, 2, 3])),              # all four resident, no accumulator pass
    ("gpt-1.3B", ([[0, 1, 2, 3]], [4, 5, 6, 7])),   # four accumulated in one pass, four folded
])
def test_full_size_resident_groups(name, schedule, progress):
    """The group schedules bench.py times (extras.resident_groups), at full size, against the
    oracle's one-at-a-time steps on the same sampled windows and the full streamed norm."""
    run_sampled_parity(name, 2, schedule=schedule, say=progress)


@pytest.mark.timeout(1100)
def test_full_size_gpt13b_twenty_steps(progress):
    """The 1.3B list's stated run: 20 steps of k = 8 at full size, each checked."""
    run_sampled_parity("gpt-1.3B", 20, say=progress)


def run_sampled_parity(name, steps, schedule=None, say=print, bench_sequence=False):
    import torch
    from harness import DeviceRun, StreamedOracle, sample_windows, compare_windows
    assert torch.cuda.is_available()
    w = configs.make(name)
    say("full-size %s: %d tensors, %d params, k=%d, schedule %s%s"
        % (name, len(w.tensors), w.total, w.k, schedule,
           ", bench.py's step sequence" if bench_sequence else ""))
    dev = DeviceRun(w, layout="flat")
    dev.schedule = schedule
    dev.device_weights = dev.first_counts = dev.separate = bench_sequence
    so = StreamedOracle(w, sample_windows(w), log=say)
    try:
        for s in range(1, steps + 1):
            scale = so.scaler.scale
            dev.step(scale)
            torch.cuda.synchronize()
            say("  device step %d done" % s)
            so.step()
            rep = compare_windows(dev, so, w)
            say("  step", s, rep)
    finally:
        dev.close()
        del dev
        torch.cuda.empty_cache()
