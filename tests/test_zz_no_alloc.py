"""mp_update_step_noalloc against mp_update_step (GPU).

The variant keeps the norm's partial sums in the library's static device array
instead of the plan's buffer; everything else is the same kernels with the same
grids, so on the same inputs it must give the same bits as mp_update_step --
state, masters, moments, 16-bit weights -- and both must meet the oracle's
parity bar.  Calls run back to back on one device, each workload after a larger
one, so the array holds the previous call's partials when the next call starts.
"""
import sys

import numpy as np
import pytest

from inputs import configs

pytestmark = pytest.mark.gpu


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


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _same_stats(sa, sb):
    assert sa.keys() == sb.keys()
    for k in sa:
        x, y = sa[k], sb[k]
        assert x == y or (x != x and y != y), (k, sa, sb)


def _same_state(a, b):
    _same_stats(a.stats(), b.stats())
    for name in ("master", "m", "v", "w16"):
        for t, (x, y) in enumerate(zip(a.host(name), b.host(name))):
            assert np.array_equal(_bits(x), _bits(y)), (name, t)


def _run_pair(mp, name, steps):
    """Steps of `name` through mp_update_step and mp_update_step_noalloc on identical
    inputs, each checked against the other bit for bit and against the oracle."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make(name)
    say("workload %s: %d tensors, %d params, k=%d" % (name, len(w.tensors), w.total, w.k))
    orc = OracleRun(w)
    ref, na = DeviceRun(w), DeviceRun(w)
    ref.one_call = na.one_call = True
    na.noalloc = True
    try:
        for s in range(1, steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            ref.step(scale)
            na.step(scale)
            _same_state(ref, na)
            rep = compare_step(na, orc, w, s)
            say("  step", s, rep)
    finally:
        ref.close()
        na.close()


def test_noalloc_matches_update_step_two_calls_shrinking(mp):
    """A larger list, then a smaller one (with an overflow step), then one micro-batch
    alone (the norm's blocks take 16 chunks each)."""
    _run_pair(mp, "llama3-8B-small", 2)
    _run_pair(mp, "edges-fp16", 3)
    _run_pair(mp, "edges-k1", 2)


def test_noalloc_refuses_plans_beyond_its_scratch(mp):
    """A plan whose norm pass takes MP_NOALLOC_MAX_NORM_BLOCKS + 1 blocks (one per chunk of
    2048 elements) is refused before anything is enqueued: the state stays as it was.  Every
    buffer of the plan is the same allocation (large enough for the fp32 views), so that
    even a wrongly accepted call would stay inside it."""
    import torch
    n = (mp.MP_NOALLOC_MAX_NORM_BLOCKS + 1) * 2048
    buf = torch.zeros(n, dtype=torch.float32, device="cuda")
    p = buf.data_ptr()
    plan = mp.mp_plan_create([n], mp.MP_BF16, [p], [p], [p], [p], [p])
    gs = mp.mp_gradset_create(plan, [p])
    st = mp.mp_state_create(mp.scaler_cfg(init_scale=1.0, enabled=False))
    try:
        info = mp.mp_plan_info(plan)
        assert info["n_chunks"] == mp.MP_NOALLOC_MAX_NORM_BLOCKS + 1, info
        before = mp.read_stats(st)
        with pytest.raises(mp.MpError) as e:
            mp.mp_update_step_noalloc(plan, st, gs, 1.0, 0, 1.0, mp.adamw_hparams())
        assert e.value.status == mp.MP_ERR_INVALID
        assert "at most" in str(e.value)
        torch.cuda.synchronize()
        _same_stats(mp.read_stats(st), before)
    finally:
        mp.mp_gradset_destroy(gs)
        mp.mp_state_destroy(st)
        mp.mp_plan_destroy(plan)
        del buf
        torch.cuda.empty_cache()
