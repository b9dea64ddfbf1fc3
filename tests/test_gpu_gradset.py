"""Gradient buffers that move between steps (needs a GPU).

A framework that frees gradients after every step hands the update new buffers
each time.  mp_gradset_update re-points the existing gradsets without
allocating; the steps must then equal the oracle exactly as with fixed buffers.
"""
import sys

import pytest

from inputs import configs

pytestmark = pytest.mark.gpu

NAN16 = 0x7FFF            # a NaN in both bf16 and fp16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mp():
    import torch
    assert torch.cuda.is_available()
    import optimizer_step_tensor_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("name", ["edges-fp16", "llama3-8B-small"])
def test_gradsets_follow_moving_buffers(mp, name):
    """Fresh gradient buffers every step, the gradsets re-pointed (each gradset's 4 staging slots
    wrap around), and the abandoned buffers filled with NaN so that a stale pointer would make
    the step overflow: every step equals the oracle."""
    import torch
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make(name)
    say("workload %s: %d tensors, k=%d, %d steps" % (name, len(w.tensors), w.k, w.steps))
    orc = OracleRun(w)
    dev = DeviceRun(w)
    try:
        for s in range(1, w.steps + 1):
            old = dev.g16
            dev.g16 = [dev.model.grad_buffers() for _ in range(w.k)]
            for gs, bufs in zip(dev.gsets, dev.g16):
                mp.mp_gradset_update(gs, bufs)
            for bufs in old:
                for x in bufs:
                    x.view(torch.int16).fill_(NAN16)
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            say("  step", s, compare_step(dev, orc, w, s))
            del old
    finally:
        dev.close()


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")   # the refused call records nothing
def test_gradset_update_errors(mp):
    import torch
    from harness import DeviceRun
    w = configs.make("edges")
    dev = DeviceRun(w)
    try:
        bufs = dev.model.grad_buffers()
        bad = list(bufs)
        bad[3] = None
        with pytest.raises(mp.MpError) as e:
            mp.mp_gradset_update(dev.gsets[0], bad)
        assert e.value.status == mp.MP_ERR_INVALID
        raw = torch.empty(4096, dtype=torch.int16, device="cuda")
        bad = list(bufs)
        bad[0] = raw.data_ptr() + 2                      # 2-byte aligned only
        with pytest.raises(mp.MpError) as e:
            mp.mp_gradset_update(dev.gsets[0], bad)
        assert e.value.status == mp.MP_ERR_ALIGN
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        torch.cuda.synchronize()
        with pytest.raises(mp.MpError) as e:            # refused while capturing
            with torch.cuda.graph(graph, stream=cap):
                mp.mp_gradset_update(dev.gsets[0], bufs)
        assert e.value.status == mp.MP_ERR_INVALID
        mp.mp_gradset_update(dev.gsets[0], bufs)        # fine outside the capture
        torch.cuda.synchronize()
    finally:
        dev.close()
