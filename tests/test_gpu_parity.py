"""Parity of the HIP library with the oracle, element by element (needs an MI355X).

Every call goes through the C ABI (the ctypes binding of include/mpstep.h).
The bar: bit-exact for the 16-bit casts, the accumulation buffer, overflow
flags, skip decisions, scaler state and optimizer clock; the global norm within
1e-5 relative; masters and moments bit-exact whenever both sides' fp32 norms
agree (else within 2e-6 relative to the magnitude of their terms).
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import inputs  # noqa: E402
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


def test_library_exports_and_device(mp):
    import torch
    say("device:", torch.cuda.get_device_name(0))
    assert mp.mp_abi_version() == 1


def test_widen_all_16bit_patterns(mp):
    import torch
    h = torch.arange(1 << 16, dtype=torch.int32, device="cuda").to(torch.int16)
    out = torch.empty(1 << 16, dtype=torch.float32, device="cuda")
    for dt in (mp.MP_BF16, mp.MP_FP16):
        mp.mp_widen_16(h.data_ptr(), out.data_ptr(), 1 << 16, dt)
        got = out.cpu().numpy()
        ref = oracle.widen16(h.cpu().numpy().view(np.uint16), dt)
        nan = np.isnan(ref)
        assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
        assert np.isnan(got[nan]).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_round_all_fp32_patterns(mp, dtype):
    """All 2^32 fp32 inputs: the device cast equals the oracle's rd16 bit for bit."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    dt = mp.MP_BF16 if dtype == "bf16" else mp.MP_FP16
    chunk = 1 << 28
    src = torch.empty(chunk, dtype=torch.int32, device="cuda")
    dst = torch.empty(chunk, dtype=torch.int16, device="cuda")
    L = oracle.lib()
    bad = 0
    for c in range((1 << 32) // chunk):
        src.copy_(torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64,
                               device="cuda").to(torch.int32))
        mp.mp_cast_to_16(src.data_ptr(), dst.data_ptr(), chunk, dt)
        got = dst.cpu().numpy().view(np.uint16)
        x = src.cpu().numpy().view(np.float32)
        parts = 16
        step = chunk // parts

        def ref(i):
            return oracle.rd16(x[i * step:(i + 1) * step], dt, L)

        with ThreadPoolExecutor(16) as ex:
            want = np.concatenate(list(ex.map(ref, range(parts))))
        bad += int((got != want).sum())
        say("cast %s chunk %d/16 mismatches so far %d" % (dtype, c + 1, bad))
    assert bad == 0


def test_generator_twins_agree(mp):
    """The device fill and the host fill of every recipe kind give the same bits."""
    import torch
    n, off = 100_003, 12_345
    recs = [inputs.recipe(inputs.key(99, 1), inputs.NORMAL, sigma=0.02),
            inputs.recipe(inputs.key(99, 2), inputs.NORMAL_TAIL, sigma=1e-4, tail_prob=0.01,
                          tail_mult=100.0),
            inputs.recipe(inputs.key(99, 3), inputs.LOGUNIF_MIX, sigma=1e-3, scale=2.0 ** 16,
                          tail_prob=0.05, lo_exp=-30, hi_exp=-20)]
    for r in recs:
        d = torch.empty(n, dtype=torch.float32, device="cuda")
        inputs.fill_dev_f32(d, r, off)
        assert np.array_equal(d.cpu().numpy().view(np.uint32),
                              inputs.gen_host_f32(n, r, off).view(np.uint32))
        for dt in (inputs.BF16, inputs.FP16):
            h = torch.empty(n, dtype=torch.int16, device="cuda")
            inputs.fill_dev_u16(h, r, dt, off)
            assert np.array_equal(h.cpu().numpy().view(np.uint16),
                                  inputs.gen_host_u16(n, r, dt, off))


PARITY = ["edges", "edges-fp16", "llama-10.5M", "gpt-124M", "gpt-1.3B-small",
          "ragged-4096-small", "llama3-8B-small"]


@pytest.mark.parametrize("name", PARITY)
def test_workload_parity(mp, name):
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make(name)
    say("workload %s: %d tensors, %d params, k=%d, %d steps"
        % (name, len(w.tensors), w.total, w.k, w.steps))
    orc = OracleRun(w)
    dev = DeviceRun(w)
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            acc_o = orc.step()
            acc_d = dev.step(scale, snapshot=True)
            rep = compare_step(dev, orc, w, s, acc_d, acc_o)
            say("  step", s, rep)
    finally:
        dev.close()


def test_one_micro_batch_on_the_edge_list(mp):
    """One bf16 micro-batch, no accumulator, on the ragged edge list (sizes 1..1000003): the
    norm pass reads the 16-bit gradient alone, each of its blocks walking 16 ragged chunks,
    and every step equals the oracle."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make("edges-k1")
    orc = OracleRun(w)
    dev = DeviceRun(w)
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            say("  step", s, compare_step(dev, orc, w, s))
    finally:
        dev.close()


@pytest.mark.parametrize("name", ["edges-fp16", "llama-10.5M"])
def test_update_step_in_one_call(mp, name):
    """mp_update_step (unscale/check/norm, AdamW, scaler in one call) equals the oracle as the
    three separate calls do, through an overflow and a change of S on the fp16 list."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make(name)
    orc = OracleRun(w)
    dev = DeviceRun(w)
    dev.one_call = True
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            say("  step", s, compare_step(dev, orc, w, s))
        with pytest.raises(mp.MpError) as e:            # bad hyper-parameters: nothing enqueued
            mp.mp_update_step(dev.model.plan, dev.state, dev.gsets[-1], 0.5, w.k == 1, 1.0,
                              mp.adamw_hparams(eps=0.0))
        assert e.value.status == mp.MP_ERR_INVALID
        with pytest.raises(mp.MpError) as e:            # so no measurement is pending either
            mp.mp_scaler_update(dev.state)
        assert e.value.status == mp.MP_ERR_ORDER
    finally:
        dev.close()


def test_random_hyperparameters(mp):
    """Eight seeded AdamW configurations far from the defaults (lr 1e-6..1, beta1 0..0.999,
    beta2 0..0.9999, eps 1e-12..1e-2, weight decay 0..0.5, clipping off or at 0.1..10) on the
    bf16 edge list: the device equals the oracle on every step of every configuration, so the
    operation order holds in every numeric regime these reach."""
    import numpy as np
    from harness import OracleRun, DeviceRun, compare_step
    rng = np.random.default_rng(2026)
    for c in range(8):
        w = configs.make("edges")
        w.hp = dict(lr=float(10 ** rng.uniform(-6, 0)), beta1=float(rng.choice([0.0, 0.5, 0.9, 0.999])),
                    beta2=float(rng.choice([0.0, 0.9, 0.999, 0.9999])),
                    eps=float(10 ** rng.uniform(-12, -2)), weight_decay=float(rng.uniform(0, 0.5)))
        w.max_norm = float(rng.choice([0.0, 0.1, 1.0, 10.0]))
        orc = OracleRun(w)
        dev = DeviceRun(w)
        try:
            for s in range(1, w.steps + 1):
                scale = orc.st.scaler.scale
                orc.step()
                dev.step(scale)
                rep = compare_step(dev, orc, w, s)
            say("  config", c, w.hp, "max_norm", w.max_norm, rep)
        finally:
            dev.close()


def test_single_micro_batch_bf16(mp):
    """bf16 with one micro-batch: no accumulator at all, the norm and AdamW read the 16-bit
    gradient directly (weight n/N = 1).  Equal to the oracle on every step."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make("llama3-8B-small")
    w.k = 1
    w.steps = 3
    orc = OracleRun(w)
    dev = DeviceRun(w)
    assert dev.model.acc is None
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            say("  step", s, compare_step(dev, orc, w, s))
    finally:
        dev.close()


def test_weight_decay_multipliers(mp):
    """Per-tensor decay multipliers ('Accumulate gradients and recompute activations': decoupled
    decay; a caller may exempt tensors): norm vectors exempt, the embedding and head at half,
    every matrix at 1.  The device equals the oracle on every step."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make("llama3-8B-small")
    w.wd_mult = [0.0 if len(shape) == 1 else (0.5 if name in ("tok_embed", "lm_head") else 1.0)
                 for name, shape in w.tensors]
    assert 0.0 in w.wd_mult and 0.5 in w.wd_mult and 1.0 in w.wd_mult
    orc = OracleRun(w)
    dev = DeviceRun(w)
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            say("  step", s, compare_step(dev, orc, w, s))
        # an exempt tensor moved by the Adam term alone: it differs from a decayed run
        t = w.wd_mult.index(0.0)
        plain = configs.make("llama3-8B-small")
        ref = OracleRun(plain)
        for _ in range(w.steps):
            ref.step()
        assert not (ref.st.masters[t] == dev.host("master")[t]).all()
    finally:
        dev.close()


def test_scaler_clamps_at_min_and_max(mp):
    """The controller's bounds ('Megatron Internals III', section 5: a floor on the scale; a cap
    on growth): S starts at 2 with growth every clean step, is capped at 4, then three overflows
    in a row halve it to 2 and 1 and hold it at the floor of 1; a clean step grows it again.  The
    device's overflow flag, skip, S and count equal the oracle's on every step."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make("edges-fp16")
    w.scaler = dict(init_scale=2.0, growth=2.0, backoff=0.5, min_scale=1.0, max_scale=4.0,
                    interval=1)
    bad_steps = (3, 4, 5)
    w.injection = lambda step: (1, 2) if step in bad_steps else None
    w.steps = 6
    orc = OracleRun(w)
    dev = DeviceRun(w)
    trace = []
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            st = dev.stats()
            assert st["found_inf"] == int(s in bad_steps) == int(orc.st.found_inf), s
            assert st["scale"] == orc.st.scaler.scale and st["good_steps"] == orc.st.scaler.good_steps
            trace.append(st["scale"])
            say("  step", s, compare_step(dev, orc, w, s))
        assert trace == [4.0, 4.0, 2.0, 1.0, 1.0, 2.0]
    finally:
        dev.close()


@pytest.mark.parametrize("name", ["edges", "edges-fp16", "gpt-1.3B-small"])
def test_unfolded_schedule(mp, name):
    """Every micro-batch accumulated first, then the norm and AdamW reading the accumulator alone
    (no last micro-batch folded in, last = NULL): the accumulator after the k-th pass and every
    step equal the oracle, in bf16 and in fp16 with an overflow."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make(name)
    orc = OracleRun(w)
    dev = DeviceRun(w)
    orc.fold_last = dev.fold_last = False
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            acc_o = orc.step()
            acc_d = dev.step(scale, snapshot=True)
            say("  step", s, compare_step(dev, orc, w, s, acc_d, acc_o))
    finally:
        dev.close()


def test_norm_is_deterministic(mp):
    """The same inputs give the same sum of squares, bit for bit, on every run."""
    from harness import DeviceRun
    w = configs.make("ragged-4096-small")
    dev = DeviceRun(w)
    try:
        dev.fill_grads(1, 1.0)
        sums = []
        for _ in range(3):
            mp.mp_unscale_check_norm(dev.model.plan, dev.state, dev.gsets[0], 0.25, 1, 1.0)
            sums.append(dev.stats()["sumsq"])
        assert sums[0] == sums[1] == sums[2]
    finally:
        dev.close()


def test_call_order_and_argument_errors(mp):
    """Structural errors are refused before anything is enqueued."""
    from harness import DeviceRun
    w = configs.make("edges")
    dev = DeviceRun(w)
    try:
        plan, st, g = dev.model.plan, dev.state, dev.gsets[0]
        with pytest.raises(mp.MpError) as e:
            mp.mp_adamw_step(plan, st, None, 1.0, 0, dev.hp)
        assert e.value.status == mp.MP_ERR_ORDER
        with pytest.raises(mp.MpError) as e:           # no measured step to decide on
            mp.mp_scaler_update(st)
        assert e.value.status == mp.MP_ERR_ORDER
        mp.mp_unscale_check_norm(plan, st, g, 0.5, 0, 1.0)
        with pytest.raises(mp.MpError) as e:           # different last micro-batch weight
            mp.mp_adamw_step(plan, st, g, 0.25, 0, dev.hp)
        assert e.value.status == mp.MP_ERR_ORDER
        mp.mp_adamw_step(plan, st, g, 0.5, 0, dev.hp)
        with pytest.raises(mp.MpError):                # nothing pending any more
            mp.mp_adamw_step(plan, st, g, 0.5, 0, dev.hp)
        for bad in (0.0, -1.0, float("nan"), float("inf")):
            with pytest.raises(mp.MpError) as e:
                mp.mp_accumulate(plan, g, bad, 1)
            assert e.value.status == mp.MP_ERR_INVALID
        hp = mp.adamw_hparams(beta1=1.0)
        mp.mp_unscale_check_norm(plan, st, g, 0.5, 0, 1.0)
        with pytest.raises(mp.MpError):
            mp.mp_adamw_step(plan, st, g, 0.5, 0, hp)
        with pytest.raises(mp.MpError) as e:
            mp.mp_state_create(mp.scaler_cfg(init_scale=3.0))
        assert e.value.status == mp.MP_ERR_INVALID
        # an accumulation after the norm changes what the norm measured
        mp.mp_unscale_check_norm(plan, st, g, 0.5, 0, 1.0)
        mp.mp_accumulate(plan, g, 0.5, 1)
        with pytest.raises(mp.MpError) as e:
            mp.mp_adamw_step(plan, st, g, 0.5, 0, dev.hp)
        assert e.value.status == mp.MP_ERR_ORDER
        # so does pointing the folded micro-batch's gradset at (other, or even the same)
        # buffers: the norm measured what the old pointers held
        mp.mp_scaler_update(st)
        mp.mp_unscale_check_norm(plan, st, g, 0.5, 0, 1.0)
        mp.mp_gradset_update(g, dev.g16[0])
        with pytest.raises(mp.MpError) as e:
            mp.mp_adamw_step(plan, st, g, 0.5, 0, dev.hp)
        assert e.value.status == mp.MP_ERR_ORDER
        with pytest.raises(mp.MpError) as e:          # the group form takes the same check
            mp.mp_adamw_step_group(plan, st, [g], [0.5], 0, dev.hp)
        assert e.value.status == mp.MP_ERR_ORDER
        # one scaler decision per measured step
        mp.mp_scaler_update(st)
        with pytest.raises(mp.MpError) as e:
            mp.mp_scaler_update(st)
        assert e.value.status == mp.MP_ERR_ORDER
        mp.mp_unscale_check_norm(plan, st, g, 0.5, 0, 1.0)
        mp.mp_adamw_step(plan, st, g, 0.5, 0, dev.hp)
        mp.mp_scaler_update(st)
    finally:
        dev.close()


def test_scaler_grows_back_after_2000_clean_steps(mp):
    """The fp16 run's controller: +inf on step 3 halves S (2^16 -> 2^15) and restarts the count;
    2000 clean steps later (step 2003) S is 2^16 again.  Device and oracle agree on every
    step's overflow flag, skip, S and count, and on the final state bit for bit."""
    from harness import OracleRun, DeviceRun, compare_step
    w = configs.make("gpt-124M-scaler")
    orc = OracleRun(w, threads=1)
    dev = DeviceRun(w)
    trace = {}
    try:
        for s in range(1, w.steps + 1):
            scale = orc.st.scaler.scale
            orc.step()
            dev.step(scale)
            st = dev.stats()
            assert st["found_inf"] == int(orc.st.found_inf), s
            assert st["scale"] == orc.st.scaler.scale and st["skipped"] == orc.st.scaler.skipped, s
            assert st["good_steps"] == orc.st.scaler.good_steps, s
            trace[s] = st["scale"]
            if s % 500 == 0:
                say("  step", s, "S", st["scale"], "count", st["good_steps"])
        assert trace[2] == 2.0 ** 16 and trace[3] == 2.0 ** 15
        assert trace[2002] == 2.0 ** 15 and trace[2003] == 2.0 ** 16
        say(compare_step(dev, orc, w, w.steps))
    finally:
        dev.close()
