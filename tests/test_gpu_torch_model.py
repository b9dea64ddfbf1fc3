"""A PyTorch model trained through the library (needs an MI355X).

The integration a training loop uses: bf16 parameters that the forward pass reads and the
step writes in place; 16-bit gradients that autograd leaves in p.grad, new buffers after
every backward, so the gradset is re-pointed for each micro-batch; micro-batches of unequal
size weighted by their share of the targets ("Accumulate gradients and recompute
activations", "Weight each mean by the targets it represents"); the last micro-batch folded
into the step with global-norm clipping ("Megatron Internals III", section 9).  In fp16 the
loss is multiplied by the dynamic loss scale before backward ("Mixed precision, loss scaling,
gradient accumulation, and activation checkpointing", section 2 "Dynamic scaling"), started
high enough that the first steps overflow, are skipped and back the scale off.  The oracle
is fed the same recorded gradient bits and must give the same masters, moments, 16-bit
weights and scaler state after every step.
"""
import types

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402


def bits16(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel().copy()


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_mlp_trained_through_the_library(fmt):
    import torch
    import optimizer_step_tensor_amd as mp
    from harness import compare_state
    assert torch.cuda.is_available()
    torch.manual_seed(20261202)
    t16 = torch.bfloat16 if fmt == "bf16" else torch.float16
    model = torch.nn.Sequential(torch.nn.Linear(96, 200), torch.nn.GELU(),
                                torch.nn.Linear(200, 24)).to("cuda", t16)
    params = list(model.parameters())
    numels = [p.numel() for p in params]
    master = [p.detach().float().contiguous() for p in params]
    m = [torch.zeros_like(x) for x in master]
    v = [torch.zeros_like(x) for x in master]
    acc = [torch.zeros_like(x) for x in master]
    scaler = (dict(init_scale=1.0, enabled=False) if fmt == "bf16" else
              dict(init_scale=2.0 ** 20, growth=2.0, backoff=0.5, interval=2, enabled=True))
    plan = mp.mp_plan_create(numels, mp.MP_BF16 if fmt == "bf16" else mp.MP_FP16, acc, master,
                             m, v, params)
    state = mp.mp_state_create(mp.scaler_cfg(**scaler))
    hpd = dict(lr=1e-2, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    hp = mp.adamw_hparams(**hpd)
    max_norm = 0.4

    dt = oracle.BF16 if fmt == "bf16" else oracle.FP16
    orc = oracle.OracleStep(dt, [x.cpu().numpy().ravel().copy() for x in master],
                            [bits16(p) for p in params], scaler=oracle.make_scaler(**scaler),
                            with_acc=True)
    schedule = [[5, 11, 16], [32, 7, 9], [13, 13, 2], [1, 40, 3], [8, 8, 8], [20, 4, 6],
                [3, 3, 30], [17, 9, 11]]
    grads = None
    skipped = committed = clipped = 0
    try:
        for step, counts in enumerate(schedule, start=1):
            k = len(counts)
            w = mp.mp_token_weights(counts)
            S = mp.read_stats(state)["scale"]
            assert S == orc.scaler.scale
            recorded = []
            for i, n in enumerate(counts):
                x = torch.randn(n, 96, device="cuda").to(t16)
                y = torch.randn(n, 24, device="cuda")
                loss = ((model(x).float() - y) ** 2).mean()       # the mean over its own rows
                (loss * S).backward()
                g = [p.grad for p in params]
                recorded.append([bits16(t) for t in g])
                if grads is None:
                    grads = mp.mp_gradset_create(plan, g)
                else:
                    mp.mp_gradset_update(grads, g)
                if i < k - 1:
                    mp.mp_accumulate(plan, grads, w[i], i == 0)
                    for p in params:
                        p.grad = None
            mp.mp_update_step(plan, state, grads, w[-1], k == 1, max_norm, hp)
            for p in params:
                p.grad = None
            torch.cuda.synchronize()

            ow = oracle.token_weights(counts)
            prev_master = [x.copy() for x in orc.masters]
            prev_m = [x.copy() for x in orc.m]
            for i in range(k - 1):
                orc.accumulate(recorded[i], ow[i], i == 0)
            orc.unscale_check_norm(recorded[-1], ow[-1], False, max_norm)
            orc.adamw_step(recorded[-1], ow[-1], False, **hpd)
            orc.scaler_update()

            stats = mp.read_stats(state)
            assert stats["found_inf"] == int(orc.found_inf), step
            assert stats["scale"] == orc.scaler.scale and stats["good_steps"] == orc.scaler.good_steps
            assert stats["skipped_total"] == orc.scaler.skipped_total
            same = orc.found_inf or np.float32(stats["grad_norm"]) == np.float32(orc.norm)
            mism = 0
            for t in range(len(params)):
                got = {"master": master[t].cpu().numpy().ravel(), "m": m[t].cpu().numpy().ravel(),
                       "v": v[t].cpu().numpy().ravel(), "w16": bits16(params[t])}
                want = {"master": orc.masters[t], "m": orc.m[t], "v": orc.v[t], "w16": orc.w16[t]}
                mism += compare_state(got, want, prev_master[t], prev_m[t],
                                      types.SimpleNamespace(hp=hpd), same, dt,
                                      " (step %d, tensor %d)" % (step, t))
            moved = any(not np.array_equal(bits16(p), o) for p, o in
                        zip(params, [oracle.rd16(x, dt) for x in prev_master]))
            if orc.found_inf:
                skipped += 1
                assert not moved, step                        # a skipped step writes nothing
            else:
                committed += 1
                clipped += stats["clip_coef"] < 1.0
                assert moved, step                            # the next forward sees the update
            print("step %d: S %g, overflow %d, norm %.6g (oracle %.6g, same bits %s), clip %.4g, "
                  "w16 mismatches %d" % (step, S, stats["found_inf"], stats["grad_norm"], orc.norm,
                                         same, stats["clip_coef"], mism), flush=True)
        assert committed >= 2 and clipped >= 1
        if fmt == "fp16":
            assert skipped >= 1
    finally:
        if grads is not None:
            mp.mp_gradset_destroy(grads)
        mp.mp_state_destroy(state)
        mp.mp_plan_destroy(plan)
