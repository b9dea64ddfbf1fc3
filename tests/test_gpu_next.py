"""The rows after the hot path: state save/restore and the sharded (ZeRO) norm (needs a GPU)."""
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


def test_state_save_restore_resumes_exactly(mp):
    """'Mixed precision ...' section 4 (state_dict round trip keeps S and the count) and pitfall 16
    (a resume that loses the count grows S late): save after step 3, restore into a state created
    with another configuration, continue -- every later step equals the uninterrupted oracle."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make("edges-fp16")            # interval 2, +inf on step 2: S moves every step
    orc = OracleRun(w)
    dev = DeviceRun(w)
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            if s == 3:
                blob = mp.save_state(dev.state)
                assert len(blob) == mp.MP_STATE_BLOB_BYTES
                mp.mp_state_destroy(dev.state)
                dev.state = mp.mp_state_create(mp.scaler_cfg(init_scale=1.0, interval=7))
                bad = bytearray(blob)
                bad[0] ^= 0xFF
                with pytest.raises(mp.MpError) as e:
                    mp.load_state(dev.state, bytes(bad))
                assert e.value.status == mp.MP_ERR_INVALID
                assert dev.stats()["scale"] == 1.0            # a refused blob changes nothing
                mp.load_state(dev.state, blob)
            say("  step", s, compare_step(dev, orc, w, s))
    finally:
        dev.close()


def _shard_plans(mp, dev, w, ranks):
    """Per-rank plans over slices of every tensor (boundaries on multiples of 8 elements)."""
    plans = []
    for r in range(ranks):
        numel, acc, master, m, v, w16, g = [], [], [], [], [], [], [[] for _ in dev.g16]
        for t, n in enumerate(w.numels):
            per = -(-n // ranks)
            per = -(-per // 8) * 8
            lo, hi = min(n, r * per), min(n, (r + 1) * per)
            if hi <= lo:
                continue
            numel.append(hi - lo)
            acc.append(dev.model.acc[t].data_ptr() + 4 * lo)
            master.append(dev.model.master[t].data_ptr() + 4 * lo)
            m.append(dev.model.m[t].data_ptr() + 4 * lo)
            v.append(dev.model.v[t].data_ptr() + 4 * lo)
            w16.append(dev.model.w16[t].data_ptr() + 2 * lo)
            for i, gl in enumerate(dev.g16):
                g[i].append(gl[t].data_ptr() + 2 * lo)
        plan = mp.mp_plan_create(numel, dev.model.dtype, acc, master, m, v, w16)
        sets = [mp.mp_gradset_create(plan, gi) for gi in g]
        plans.append((plan, sets))
    return plans


@pytest.mark.parametrize("name", ["llama3-8B-small", "edges", "edges-fp16"])
def test_sharded_norm_matches_unsharded(mp, name):
    """'Megatron Internals III' sections 6 and 9 / 'Your weights fit...' (ZeRO): four ranks' slices,
    each with its own plan and state replica; one reduction of the partial sums of squares gives
    every rank the global norm and the same skip decision; the result is the unsharded update."""
    run_sharded(mp, name, grouped=False)


@pytest.mark.parametrize("name", ["edges-fp16", "llama-10.5M"])
def test_sharded_norm_with_resident_groups(mp, name):
    """The same four ranks, each folding all of its resident micro-batches into the partial norm
    and the AdamW pass as one group (mp_norm_partial_group, mp_adamw_step_group): still the
    unsharded one-at-a-time update, bit for bit, through the fp16 list's overflow."""
    run_sharded(mp, name, grouped=True)


def run_sharded(mp, name, grouped):
    import torch
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make(name)
    ranks = 4
    orc = OracleRun(w)
    dev = DeviceRun(w)
    plans = _shard_plans(mp, dev, w, ranks)
    cfg = (mp.scaler_cfg(**w.scaler) if w.scaler is not None
           else mp.scaler_cfg(init_scale=1.0, enabled=False))
    states = [mp.mp_state_create(cfg) for _ in plans]
    partials = torch.zeros(ranks, dtype=torch.float64, device="cuda")
    total = torch.zeros(1, dtype=torch.float64, device="cuda")
    try:
        for s in range(1, 4):                  # edges-fp16 overflows on step 2: every rank skips
            scale = orc.st.scaler.scale
            orc.step()
            dev.fill_grads(s, scale)
            wts = mp.mp_token_weights(w.token_counts(s))
            for r, (plan, sets) in enumerate(plans):
                if grouped:
                    mp.mp_norm_partial_group(plan, states[r], sets, wts, 1,
                                             partials.data_ptr() + 8 * r)
                    continue
                for i in range(w.k - 1):
                    mp.mp_accumulate(plan, sets[i], wts[i], i == 0)
                mp.mp_norm_partial(plan, states[r], sets[-1], wts[-1], 0,
                                   partials.data_ptr() + 8 * r)
            # stands in for the all-reduce: the ranks' partial sums added in rank order
            host = partials.cpu().numpy()
            acc_sum = 0.0
            for r in range(ranks):
                acc_sum = acc_sum + float(host[r])
            total.fill_(acc_sum)
            for r, (plan, sets) in enumerate(plans):
                mp.mp_norm_finish(plan, states[r], total.data_ptr(), w.max_norm)
                if grouped:
                    mp.mp_adamw_step_group(plan, states[r], sets, wts, 1, dev.hp)
                else:
                    mp.mp_adamw_step(plan, states[r], sets[-1], wts[-1], 0, dev.hp)
                mp.mp_scaler_update(states[r])
            # every rank holds the same scalars; compare the full tensors with the oracle
            stats = [mp.read_stats(st) for st in states]
            assert all(x == stats[0] for x in stats)

            class RankView:                    # rank 0's scalars, the full tensors
                torch = dev.torch
                host = staticmethod(dev.host)
                stats = staticmethod(lambda: stats[0])

            say("  step", s, compare_step(RankView, orc, w, s))
        with pytest.raises(mp.MpError) as e:       # finish without a partial
            mp.mp_norm_finish(plans[0][0], states[0], total.data_ptr(), 1.0)
        assert e.value.status == mp.MP_ERR_ORDER
    finally:
        for plan, sets in plans:
            for g in sets:
                mp.mp_gradset_destroy(g)
            mp.mp_plan_destroy(plan)
        for st in states:
            mp.mp_state_destroy(st)
        dev.close()


@pytest.mark.parametrize("name", ["llama3-8B-small", "edges-fp16"])
def test_flattened_buffers(mp, name):
    """'Megatron Internals III' section 8 (flattened fp32 main-gradient buffers): the model's
    buffers as one contiguous allocation per kind with per-tensor views -- same results as the
    oracle, bit for bit."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make(name)
    orc = OracleRun(w)
    dev = DeviceRun(w, layout="flat")
    try:
        for s in range(1, min(w.steps, 3) + 1):
            scale = orc.st.scaler.scale
            acc_o = orc.step()
            acc_d = dev.step(scale, snapshot=True)
            say("  step", s, compare_step(dev, orc, w, s, acc_d, acc_o))
    finally:
        dev.close()


def test_whole_model_as_one_tensor(mp):
    """A caller who flattens the whole model into one buffer per kind passes a one-tensor plan
    (the chunk table then cuts one range): masters, moments and 16-bit weights equal the
    per-tensor oracle's, bit for bit when the norms agree, else within the parity bar."""
    import torch
    import inputs
    from harness import OracleRun, compare_state, oracle_dtype
    w = configs.make("llama3-8B-small")
    orc = OracleRun(w)
    total = w.total
    offs = np.cumsum([0] + w.numels[:-1])
    bufs = {name: torch.zeros(total, dtype=torch.float32, device="cuda")
            for name in ("acc", "master", "m", "v")}
    w16 = torch.zeros(total, dtype=torch.bfloat16, device="cuda")
    g16 = [torch.zeros(total, dtype=torch.bfloat16, device="cuda") for _ in range(w.k)]
    for t, (o, n) in enumerate(zip(offs, w.numels)):
        inputs.fill_dev_f32(bufs["master"][o:o + n], w.master_recipe(t))
    plan = mp.mp_plan_create([total], mp.MP_BF16, [bufs["acc"]], [bufs["master"]], [bufs["m"]],
                             [bufs["v"]], [w16])
    sets = [mp.mp_gradset_create(plan, [g]) for g in g16]
    st = mp.mp_state_create(mp.scaler_cfg(init_scale=1.0, enabled=False))
    hp = mp.adamw_hparams(**w.hp)
    try:
        for s in range(1, 3):
            orc.step()
            for i in range(w.k):
                for t, (o, n) in enumerate(zip(offs, w.numels)):
                    inputs.fill_dev_u16(g16[i][o:o + n], w.grad_recipe(s, i, t), w.dtype)
            wts = mp.mp_token_weights(w.token_counts(s))
            for i in range(w.k - 1):
                mp.mp_accumulate(plan, sets[i], wts[i], i == 0)
            mp.mp_unscale_check_norm(plan, st, sets[-1], wts[-1], 0, w.max_norm)
            mp.mp_adamw_step(plan, st, sets[-1], wts[-1], 0, hp)
            mp.mp_scaler_update(st)
            stats = mp.read_stats(st)
            assert stats["found_inf"] == 0 and stats["step"] == orc.st.clock.t
            assert abs(stats["grad_norm"] - orc.st.norm) <= 1e-5 * orc.st.norm
            same = (np.float32(stats["grad_norm"]) == np.float32(orc.st.norm)
                    and np.float32(stats["clip_coef"]) == np.float32(orc.st.coef))
            host = {name: bufs[name].cpu().numpy() for name in ("master", "m", "v")}
            host["w16"] = w16.cpu().view(torch.int16).numpy().view(np.uint16)
            mism = 0
            for t, (o, n) in enumerate(zip(offs, w.numels)):
                got = {name: a[o:o + n] for name, a in host.items()}
                want = {"master": orc.st.masters[t], "m": orc.st.m[t], "v": orc.st.v[t],
                        "w16": orc.st.w16[t]}
                mism += compare_state(got, want, orc.prev_master[t], orc.prev_m[t], w, same,
                                      oracle_dtype(w), " (tensor %d)" % t)
            say("  step", s, "norm", stats["grad_norm"], "same bits", bool(same),
                "w16 mismatches", mism)
    finally:
        for g in sets:
            mp.mp_gradset_destroy(g)
        mp.mp_state_destroy(st)
        mp.mp_plan_destroy(plan)
