"""Token weights computed and read on the device (needs an MI355X).

The weights of "Accumulate gradients and recompute activations", section "Weight each mean by
the targets it represents", from counts that stay in device memory: mp_token_weights_dev must
give the host call's bits, the group entry points reading those weights on the device must step
exactly as the host-weight calls do, counts the host would refuse must turn into a skipped step,
and a captured graph must read the counts of each replay.
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


def device_weights(mp, counts):
    import torch
    c = torch.tensor(counts, dtype=torch.int64, device="cuda")
    w = torch.full((len(counts),), 7.0, dtype=torch.float32, device="cuda")
    mp.mp_token_weights_dev(len(counts), c, w)
    return w.cpu().numpy()


def test_device_weights_equal_the_oracle(mp):
    """fp32(n_i / N) bit for bit, for k up to beyond one block of threads and totals up to 2^53."""
    rng = np.random.default_rng(44)
    cases = [list(rng.integers(1, 10 ** 6, k)) for k in (1, 2, 3, 4, 8, 31, 256, 257, 1000)]
    cases += [[2 ** 52, 2 ** 52], [2 ** 53 - 1, 1], [1] * 3, [3, 2 ** 40, 7]]
    for counts in cases:
        got = device_weights(mp, counts)
        ref = oracle.token_weights(counts)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), counts[:4]
        assert np.array_equal(got, np.array(mp.mp_token_weights(counts), np.float32))


def test_refused_counts_give_nan_weights(mp):
    """Counts the host call refuses (a micro-batch without targets, N > 2^53) cannot be refused
    on the device without a sync: every weight comes out NaN instead."""
    for counts in ([4, 0], [0], [-3, 5, 6], [2 ** 53, 1], [2 ** 62, 2 ** 62, 1], [1, 2, -(2 ** 63)]):
        with pytest.raises(ValueError):
            oracle.token_weights(counts)
        got = device_weights(mp, counts)
        assert np.isnan(got).all(), counts


@pytest.mark.parametrize("name,fold_last,sequence", [
    ("edges-fp16", True, "weights_dev"), ("llama-10.5M", True, "weights_dev"),
    ("edges", False, "weights_dev"),
    ("edges-fp16", True, "bench_eager"), ("llama-10.5M", True, "bench_eager"),
    ("llama-10.5M", True, "bench_graph"), ("edges", False, "counts_in_first")])
def test_device_weight_steps_equal_the_oracle(mp, name, fold_last, sequence):
    """Steps whose weights come from device counts equal the oracle's, through the fp16 list's
    overflow and change of S: weights from mp_token_weights_dev, or computed inside the first
    accumulation (mp_accumulate_first_counts); then one-micro-batch group calls reading them on
    the device -- mp_update_step_group, or (bench_eager, bench.py's eager step) the norm, AdamW
    and scaler as three calls."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make(name)
    orc = OracleRun(w)
    dev = DeviceRun(w)
    orc.fold_last = dev.fold_last = fold_last
    dev.device_weights = True
    dev.first_counts = sequence != "weights_dev"
    dev.separate = sequence == "bench_eager"
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            say("  step", s, compare_step(dev, orc, w, s))
    finally:
        dev.close()


@pytest.mark.parametrize("in_first", [False, True])
def test_refused_counts_skip_the_step(mp, in_first):
    """A count of zero on the device makes the weights NaN, so the step is skipped exactly as an
    overflow is ("Discard a failed partial logical update"): no master, moment or 16-bit weight
    changes, the clock stays, and the scaler backs off -- with the weights from
    mp_token_weights_dev or computed inside the first accumulation."""
    import torch
    from harness import DeviceRun
    w = configs.make("edges-fp16")
    dev = DeviceRun(w)
    dev.device_weights = True
    try:
        dev.step(w.scaler["init_scale"])
        before = dev.stats()
        assert before["skipped"] == 0
        snap = {n: [x.clone() for x in getattr(dev.model, n)] for n in ("master", "m", "v", "w16")}
        dev.fill_grads(2, before["scale"])
        cnt = torch.tensor([0] + [5] * (w.k - 1), dtype=torch.int64, device="cuda")
        wts = torch.empty(w.k, dtype=torch.float32, device="cuda")
        plan = dev.model.plan
        if not in_first:
            mp.mp_token_weights_dev(w.k, cnt, wts)
        for i in range(w.k - 1):
            if in_first and i == 0:
                mp.mp_accumulate_first_counts(plan, [dev.gsets[0]], w.k, cnt, wts)
            else:
                mp.mp_accumulate_group(plan, [dev.gsets[i]], wts.data_ptr() + 4 * i, i == 0)
        mp.mp_update_step_group(plan, dev.state, [dev.gsets[-1]], wts.data_ptr() + 4 * (w.k - 1),
                                w.k == 1, w.max_norm, dev.hp)
        after = dev.stats()
        say("  after refused counts:", after)
        assert after["found_inf"] == 1 and after["skipped"] == 1
        assert after["step"] == before["step"]
        assert after["skipped_total"] == before["skipped_total"] + 1
        assert after["good_steps"] == 0
        assert after["scale"] == max(before["scale"] * w.scaler["backoff"], w.scaler["min_scale"])
        assert after["beta1_pow"] == before["beta1_pow"]
        for n, xs in snap.items():
            for x, y in zip(xs, getattr(dev.model, n)):
                assert torch.equal(x.view(torch.int16 if n == "w16" else torch.int32),
                                   y.view(torch.int16 if n == "w16" else torch.int32)), n
    finally:
        dev.close()


@pytest.mark.parametrize("bench_graph", [False, True])
def test_graph_replays_read_each_replays_counts(mp, bench_graph):
    """A captured step (device weights, accumulation, update) replayed with new counts written
    into the same device buffer between replays equals eager steps with host weights of those
    counts, bit for bit, on every replay.  bench_graph: bench.py's captured step (the weights
    computed inside the first accumulation, then mp_update_step_group); else
    mp_token_weights_dev and the norm, AdamW and scaler as three calls."""
    import torch
    from harness import DeviceRun
    w = configs.make("llama-10.5M")
    eager, graphed = DeviceRun(w), DeviceRun(w)
    k = w.k
    cnt = torch.ones(k, dtype=torch.int64, device="cuda")
    wts = torch.empty(k, dtype=torch.float32, device="cuda")
    wp = [wts.data_ptr() + 4 * i for i in range(k)]

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        st = torch.cuda.current_stream()
        plan = graphed.model.plan
        if not bench_graph:
            mp.mp_token_weights_dev(k, cnt, wts, st)
        for i in range(k - 1):
            if bench_graph and i == 0:
                mp.mp_accumulate_first_counts(plan, [graphed.gsets[0]], k, cnt, wts, st)
            else:
                mp.mp_accumulate_group(plan, [graphed.gsets[i]], wp[i], i == 0, st)
        if bench_graph:
            mp.mp_update_step_group(plan, graphed.state, [graphed.gsets[-1]], wp[-1], 0,
                                    w.max_norm, graphed.hp, st)
        else:
            # the separate norm and AdamW calls, each reading the last weight on the device
            mp.mp_unscale_check_norm_group(plan, graphed.state, [graphed.gsets[-1]], wp[-1], 0,
                                           w.max_norm, st)
            mp.mp_adamw_step_group(plan, graphed.state, [graphed.gsets[-1]], wp[-1], 0,
                                   graphed.hp, st)
            mp.mp_scaler_update(graphed.state, st)
    try:
        for r in range(1, 5):
            counts = w.token_counts(r)
            eager.fill_grads(r, 1.0)
            graphed.fill_grads(r, 1.0)
            cnt.copy_(torch.tensor(counts, dtype=torch.int64))
            torch.cuda.synchronize()
            weights = mp.mp_token_weights(counts)
            plan = eager.model.plan
            for i in range(k - 1):
                mp.mp_accumulate(plan, eager.gsets[i], weights[i], i == 0)
            mp.mp_update_step(plan, eager.state, eager.gsets[-1], weights[-1], 0, w.max_norm,
                              eager.hp)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(wts.cpu().numpy(), np.array(weights, np.float32)), r
            a, b = eager.stats(), graphed.stats()
            assert a == b and a["step"] == r
            for name in ("acc", "master", "m", "v"):
                for x, y in zip(getattr(eager.model, name), getattr(graphed.model, name)):
                    assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (r, name)
            for x, y in zip(eager.model.w16, graphed.model.w16):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (r, "w16")
            say("  replay", r, "counts", counts)
    finally:
        del g
        eager.close()
        graphed.close()



@pytest.mark.parametrize("n", [1, 2, 4])
def test_first_accumulation_with_counts(mp, n):
    """mp_accumulate_first_counts: one pass gives the bits of mp_token_weights_dev followed by
    mp_accumulate_group(first=1) -- the weights it writes for the later passes (equal to the
    oracle's) and the accumulator -- for valid counts, for the largest k, and for counts the
    host would refuse (NaN weights, NaN accumulator)."""
    import torch
    import inputs
    from harness import DeviceRun
    w = configs.make("edges")
    dev = DeviceRun(w, sep_grads=False)
    extra = [dev.model.grad_buffers() for _ in range(n - 1)]
    sets = [dev.gsets[0]] + [dev.model.gradset(g) for g in extra]
    try:
        for i, gl in enumerate([dev.g16[0]] + extra):
            for t, x in enumerate(gl):
                inputs.fill_dev_u16(x, w.grad_recipe(1, i, t), w.dtype)
        valid = [451, 402, 509, 433, 500, 470][:max(n, 3)]
        for counts in (valid, [7] * 64, [4, 0, 5, 6][:max(n, 3)]):
            k = len(counts)
            c = torch.tensor(counts, dtype=torch.int64, device="cuda")
            w_ref = torch.full((k,), 3.0, dtype=torch.float32, device="cuda")
            mp.mp_token_weights_dev(k, c, w_ref)
            mp.mp_accumulate_group(dev.model.plan, sets, w_ref.data_ptr(), True)
            acc_ref = [a.cpu().numpy().copy() for a in dev.model.acc]
            for a in dev.model.acc:
                a.fill_(5.0)
            w_got = torch.full((k,), 3.0, dtype=torch.float32, device="cuda")
            mp.mp_accumulate_first_counts(dev.model.plan, sets, k, c, w_got)
            acc_got = [a.cpu().numpy() for a in dev.model.acc]
            got = w_got.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), w_ref.cpu().numpy().view(np.uint32)), counts
            if 0 not in counts:
                want = np.asarray(oracle.token_weights(counts), dtype=np.float32)
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), counts
            else:
                assert np.isnan(got).all() and all(np.isnan(a).all() for a in acc_got)
            for a, b in zip(acc_got, acc_ref):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), counts
            say("  n=%d k=%d ok (weights %s)" % (n, k, got[:3]))
        c = torch.ones(65, dtype=torch.int64, device="cuda")
        w_got = torch.empty(65, dtype=torch.float32, device="cuda")
        with pytest.raises(mp.MpError) as e:                  # k out of range
            mp.mp_accumulate_first_counts(dev.model.plan, sets, 65, c, w_got)
        assert e.value.status == mp.MP_ERR_INVALID
        with pytest.raises(mp.MpError) as e:                  # fewer counts than gradsets
            mp.mp_accumulate_first_counts(dev.model.plan, sets, n - 1, c, w_got)
        assert e.value.status == mp.MP_ERR_INVALID
        with pytest.raises(mp.MpError) as e:                  # misaligned counts
            mp.mp_accumulate_first_counts(dev.model.plan, sets, n, c.data_ptr() + 4, w_got)
        assert e.value.status == mp.MP_ERR_ALIGN
    finally:
        for g in sets[1:]:
            mp.mp_gradset_destroy(g)
        dev.close()
