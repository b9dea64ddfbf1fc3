"""The step is stream-ordered with no host synchronisation, so a whole step can be captured in a
HIP graph (through torch.cuda.graph) and replayed (needs a GPU).  Every replay is checked
against the same step run eagerly, with eager work and synchronisations between replays."""
import pytest

from inputs import configs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("form", ["separate calls", "mp_update_step"])
def test_graph_replays_equal_eager_steps(form):
    import torch
    import optimizer_step_tensor_amd as mp
    from harness import DeviceRun
    w = configs.make("llama-10.5M")
    eager, graphed = DeviceRun(w), DeviceRun(w)
    weights = mp.mp_token_weights(w.token_counts(1))
    k = w.k

    def step(dev, stream):
        plan = dev.model.plan
        for i in range(k - 1):
            mp.mp_accumulate(plan, dev.gsets[i], weights[i], i == 0, stream)
        if form == "mp_update_step":
            mp.mp_update_step(plan, dev.state, dev.gsets[-1], weights[-1], 0, w.max_norm, dev.hp,
                              stream)
            return
        mp.mp_unscale_check_norm(plan, dev.state, dev.gsets[-1], weights[-1], 0, w.max_norm, stream)
        mp.mp_adamw_step(plan, dev.state, dev.gsets[-1], weights[-1], 0, dev.hp, stream)
        mp.mp_scaler_update(dev.state, stream)

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        step(graphed, torch.cuda.current_stream())
    try:
        for r in range(1, 5):
            eager.fill_grads(r, 1.0)           # eager work between replays
            graphed.fill_grads(r, 1.0)
            torch.cuda.synchronize()
            step(eager, None)
            g.replay()
            torch.cuda.synchronize()
            a, b = eager.stats(), graphed.stats()
            assert a == b and a["step"] == r
            for name in ("acc", "master", "m", "v"):
                for x, y in zip(getattr(eager.model, name), getattr(graphed.model, name)):
                    assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (r, name)
            for x, y in zip(eager.model.w16, graphed.model.w16):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (r, "w16")
    finally:
        del g
        eager.close()
        graphed.close()


def test_graph_replays_follow_the_scaler():
    """One captured step on the fp16 edge list (dynamic S, growth every 2 clean steps, an inf at
    step 2), replayed for every step with new gradients and new device token counts written
    between replays: each replay equals the oracle's step, through the skip, the backoff and
    the growth, so the scaler's decisions live on the device and nothing captured goes stale."""
    import torch
    import optimizer_step_tensor_amd as mp
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make("edges-fp16")
    orc, dev = OracleRun(w), DeviceRun(w)
    k = w.k
    cnt = torch.ones(k, dtype=torch.int64, device="cuda")
    wts = torch.empty(k, dtype=torch.float32, device="cuda")
    wp = [wts.data_ptr() + 4 * i for i in range(k)]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        st = torch.cuda.current_stream()
        plan = dev.model.plan
        mp.mp_token_weights_dev(k, cnt, wts, st)
        for i in range(k - 1):
            mp.mp_accumulate_group(plan, [dev.gsets[i]], wp[i], i == 0, st)
        mp.mp_update_step_group(plan, dev.state, [dev.gsets[-1]], wp[-1], 0, w.max_norm, dev.hp,
                                st)
    try:
        seen = set()
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            assert dev.stats()["scale"] == scale
            orc.step()
            dev.fill_grads(s, scale)
            cnt.copy_(torch.tensor(w.token_counts(s), dtype=torch.int64))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            rep = compare_step(dev, orc, w, s)
            seen.add("skip" if rep["found_inf"] else "clean")
            print("  replay", s, rep, flush=True)
        assert seen == {"skip", "clean"}
        assert dev.stats()["scale"] != w.scaler["init_scale"]
    finally:
        del g
        dev.close()


def test_graph_replays_of_a_resident_group_step():
    """A captured step that folds all four resident micro-batches into the norm and AdamW passes
    (no accumulator pass), with the weights computed on the device from a count buffer rewritten
    between replays, equals the same group step run eagerly with host weights, bit for bit, on
    every replay."""
    import numpy as np
    import torch
    import optimizer_step_tensor_amd as mp
    from harness import DeviceRun
    w = configs.make("llama-10.5M")
    eager, graphed = DeviceRun(w), DeviceRun(w)
    k = w.k
    cnt = torch.ones(k, dtype=torch.int64, device="cuda")
    wts = torch.empty(k, dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        st = torch.cuda.current_stream()
        mp.mp_token_weights_dev(k, cnt, wts, st)
        mp.mp_update_step_group(graphed.model.plan, graphed.state, graphed.gsets, wts, 1,
                                w.max_norm, graphed.hp, st)
    try:
        for r in range(1, 5):
            counts = w.token_counts(r)
            eager.fill_grads(r, 1.0)
            graphed.fill_grads(r, 1.0)
            cnt.copy_(torch.tensor(counts, dtype=torch.int64))
            torch.cuda.synchronize()
            mp.mp_update_step_group(eager.model.plan, eager.state, eager.gsets,
                                    mp.mp_token_weights(counts), 1, w.max_norm, eager.hp)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(wts.cpu().numpy(),
                                  np.array(mp.mp_token_weights(counts), np.float32)), r
            a, b = eager.stats(), graphed.stats()
            assert a == b and a["step"] == r
            for name in ("master", "m", "v"):
                for x, y in zip(getattr(eager.model, name), getattr(graphed.model, name)):
                    assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (r, name)
            for x, y in zip(eager.model.w16, graphed.model.w16):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (r, "w16")
    finally:
        del g
        eager.close()
        graphed.close()
