"""Resident micro-batches folded in groups (needs an MI355X).

When the 16-bit gradients of several micro-batches are in device memory at once, one pass can
fold them all in ("Mixed precision ...", section 2 "Gradient accumulation"; "Accumulate
gradients and recompute activations", "Weight each mean by the targets it represents"): the
running sum stays in a register and each term is added with the roundings of one accumulation
step, so every schedule of groups must give the bits of the one-at-a-time accumulation.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from inputs import configs  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mp():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import optimizer_step_tensor_amd as m
    m.lib()
    return m


def _same_values(got, ref):
    """Equal bits where the oracle is finite, the same inf/NaN pattern elsewhere."""
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isposinf(got), np.isposinf(ref))
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_accumulate_group_equals_the_oracle(mp, dtype):
    """Every 16-bit pattern (infinities, NaNs, signed zeros and subnormals included) on ragged
    tensors: groups of 1-4 micro-batches, with and without `first`, against the oracle's
    one-by-one accumulation."""
    import torch
    dt = mp.MP_BF16 if dtype == "bf16" else mp.MP_FP16
    odt = oracle.BF16 if dtype == "bf16" else oracle.FP16
    rng = np.random.default_rng(7 if dtype == "bf16" else 8)
    numels = [1, 3, 4, 5, 2047, 2049, 4096, 70001]
    model = mp.ModelState(numels, dt, with_acc=True)
    grads = [model.grad_buffers() for _ in range(4)]
    sets = [model.gradset(g) for g in grads]
    host_g = [[rng.integers(0, 1 << 16, n).astype(np.uint16) for n in numels] for _ in range(4)]
    for g, hg in zip(grads, host_g):
        for x, h in zip(g, hg):
            x.view(torch.int16).copy_(torch.from_numpy(h.view(np.int16)))
    try:
        for n in (1, 2, 3, 4):
            for first in (True, False):
                w = [float(np.float32(rng.uniform(0.01, 1.0))) for _ in range(n)]
                acc0 = [rng.normal(0, 1, m).astype(np.float32) for m in numels]
                for a, h in zip(model.acc, acc0):
                    a.copy_(torch.from_numpy(h))
                mp.mp_accumulate_group(model.plan, sets[:n], w, first)
                torch.cuda.synchronize()
                for t, m in enumerate(numels):
                    ref = acc0[t].copy()
                    for i in range(n):
                        oracle.accumulate_tensor(host_g[i][t], ref, odt, w[i], first and i == 0)
                    _same_values(model.acc[t].cpu().numpy(), ref)
                say("  n", n, "first", first, "ok")
    finally:
        for s_ in sets:
            mp.mp_gradset_destroy(s_)
        model.close()


CASES = [
    ("edges", [[0, 1]], [2]),
    ("edges", [], [0, 1, 2]),
    ("edges", [[0]], [1, 2]),
    ("edges-fp16", [], [0, 1]),
    ("llama-10.5M", [[0, 1]], [2, 3]),
    ("llama-10.5M", [], [0, 1, 2, 3]),
    ("gpt-1.3B-small", [[0, 1, 2, 3]], [4, 5, 6, 7]),
    ("gpt-1.3B-small", [[0, 1, 2], [3, 4, 5]], [6, 7]),
    ("gpt-1.3B-small", [[0], [1, 2, 3, 4]], [5, 6, 7]),
]


@pytest.mark.parametrize("name,acc_groups,fold", CASES,
                         ids=["%s-%s-%s" % (c[0], c[1], c[2]) for c in CASES])
def test_group_schedules_equal_the_oracle(mp, name, acc_groups, fold):
    """Whole steps with the micro-batches folded in groups equal the oracle's one-at-a-time
    steps, through the fp16 list's overflow and change of S."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make(name)
    orc = OracleRun(w)
    dev = DeviceRun(w)
    dev.schedule = (acc_groups, fold)
    try:
        for s in range(1, min(w.steps, 4) + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            say("  step", s, compare_step(dev, orc, w, s))
    finally:
        dev.close()


def test_group_schedule_with_device_weights(mp):
    """The group calls reading their weights from mp_token_weights_dev's output."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make("edges-fp16")
    orc = OracleRun(w)
    dev = DeviceRun(w)
    dev.schedule = ([[0]], [1])
    dev.device_weights = True
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            say("  step", s, compare_step(dev, orc, w, s))
    finally:
        dev.close()


def test_group_argument_errors(mp):
    """Out-of-range groups, foreign gradsets and plans without accumulators are refused before
    anything is enqueued; the separate AdamW call does not accept a group's measurement."""
    from harness import DeviceRun
    w = configs.make("edges")
    dev = DeviceRun(w)
    other = DeviceRun(w)
    plan, st = dev.model.plan, dev.state
    try:
        for sets, wts, code in (
                (dev.gsets * 2, [0.2] * 6, mp.MP_ERR_INVALID),        # more than 4
                ([dev.gsets[0], other.gsets[1]], [0.5, 0.5], mp.MP_ERR_INVALID),
                ([dev.gsets[0]], [float("nan")], mp.MP_ERR_INVALID),
                ([dev.gsets[0]], [0.0], mp.MP_ERR_INVALID)):
            with pytest.raises(mp.MpError) as e:
                mp.mp_accumulate_group(plan, sets, wts, True)
            assert e.value.status == code
            with pytest.raises(mp.MpError) as e:
                mp.mp_update_step_group(plan, st, sets, wts, True, 1.0, dev.hp)
            assert e.value.status == code
        with pytest.raises(mp.MpError) as e:
            mp.mp_accumulate_group(plan, [], [], True)
        assert e.value.status == mp.MP_ERR_INVALID
        with pytest.raises(mp.MpError) as e:                     # misaligned device weights
            mp.mp_accumulate_group(plan, dev.gsets[:2], 0x10002, True)
        assert e.value.status == mp.MP_ERR_ALIGN
        # nothing was measured, so the scaler has no decision to take
        with pytest.raises(mp.MpError) as e:
            mp.mp_scaler_update(st)
        assert e.value.status == mp.MP_ERR_ORDER
        # a norm over one micro-batch does not license an AdamW step over another
        mp.mp_unscale_check_norm(plan, st, dev.gsets[2], 0.3, 0, 1.0)
        with pytest.raises(mp.MpError) as e:
            mp.mp_adamw_step(plan, st, dev.gsets[1], 0.3, 0, dev.hp)
        assert e.value.status == mp.MP_ERR_ORDER
        mp.mp_adamw_step(plan, st, dev.gsets[2], 0.3, 0, dev.hp)
        mp.mp_scaler_update(st)
    finally:
        dev.close()
        other.close()
    # a plan without accumulators takes a group only as the whole update
    w1 = configs.make("edges")
    m = mp.ModelState(w1.numels, mp.MP_BF16, with_acc=False)
    g = [m.gradset(m.grad_buffers()) for _ in range(2)]
    state = mp.mp_state_create(mp.scaler_cfg(init_scale=1.0, enabled=False))
    try:
        with pytest.raises(mp.MpError) as e:
            mp.mp_accumulate_group(m.plan, g, [0.5, 0.5], True)
        assert e.value.status == mp.MP_ERR_INVALID
        with pytest.raises(mp.MpError) as e:
            mp.mp_update_step_group(m.plan, state, g, [0.5, 0.5], False, 1.0, mp.adamw_hparams())
        assert e.value.status == mp.MP_ERR_INVALID
    finally:
        for x in g:
            mp.mp_gradset_destroy(x)
        mp.mp_state_destroy(state)
        m.close()


def test_group_with_refused_device_counts_skips(mp):
    """A resident group whose device weights come from counts the host call would refuse (a
    micro-batch without targets) folds NaN weights in, so the step overflows and is skipped:
    nothing written, the clock kept, S backed off."""
    import torch
    from harness import DeviceRun
    w = configs.make("edges-fp16")
    dev = DeviceRun(w)
    try:
        dev.fill_grads(1, w.scaler["init_scale"])
        before = dev.stats()
        snap = [x.clone() for x in dev.model.master]
        cnt = torch.tensor([5] * (w.k - 1) + [0], dtype=torch.int64, device="cuda")
        wts = torch.empty(w.k, dtype=torch.float32, device="cuda")
        mp.mp_token_weights_dev(w.k, cnt, wts)
        mp.mp_update_step_group(dev.model.plan, dev.state, dev.gsets, wts, True, w.max_norm,
                                dev.hp)
        after = dev.stats()
        assert after["found_inf"] == 1 and after["skipped"] == 1 and after["step"] == 0
        assert after["scale"] == before["scale"] * w.scaler["backoff"]
        for x, y in zip(snap, dev.model.master):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    finally:
        dev.close()


def test_group_with_a_repeated_micro_batch(mp):
    """A gradset may appear twice in a group: the fold adds it twice, exactly as two
    one-by-one accumulations of it do."""
    import torch
    from harness import DeviceRun
    w = configs.make("edges")
    a, b = DeviceRun(w), DeviceRun(w)
    try:
        for run in (a, b):
            run.fill_grads(1, 1.0)
        mp.mp_accumulate_group(a.model.plan, [a.gsets[0], a.gsets[1], a.gsets[0]],
                               [0.25, 0.5, 0.25], True)
        mp.mp_accumulate(b.model.plan, b.gsets[0], 0.25, True)
        mp.mp_accumulate(b.model.plan, b.gsets[1], 0.5, False)
        mp.mp_accumulate(b.model.plan, b.gsets[0], 0.25, False)
        torch.cuda.synchronize()
        for x, y in zip(a.model.acc, b.model.acc):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    finally:
        a.close()
        b.close()
