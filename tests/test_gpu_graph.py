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
