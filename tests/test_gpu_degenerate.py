"""Degenerate values through the whole step, device against oracle (needs a GPU).

Hand-made inputs rather than the generator: bf16 gradients whose accumulation
overflows fp32, gradients and moments deep in the fp32 subnormal range (the
device must not flush denormals), all-zero gradients (decay only), a NaN, and
the fp16 format's extremes.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


@pytest.fixture(scope="module")
def mp():
    import torch
    assert torch.cuda.is_available()
    import optimizer_step_tensor_amd as m
    m.lib()
    return m


def run_both(mp, dtype, masters, grads, counts, steps=2, max_norm=1.0, scaler=None,
             m0=None, v0=None):
    """grads[step][micro] is a list of uint16 arrays (one per tensor)."""
    import torch
    numels = [x.size for x in masters]
    k = len(grads[0])
    odt = oracle.BF16 if dtype == mp.MP_BF16 else oracle.FP16
    sc = oracle.make_scaler(**scaler) if scaler else oracle.make_scaler(init_scale=1.0, enabled=False)
    orc = oracle.OracleStep(odt, [x.copy() for x in masters], [oracle.rd16(x, odt) for x in masters],
                            m=[x.copy() for x in m0] if m0 else None,
                            v=[x.copy() for x in v0] if v0 else None,
                            scaler=sc, with_acc=k > 1)
    model = mp.ModelState(numels, dtype, with_acc=k > 1)
    for t in range(len(numels)):
        model.master[t].copy_(torch.from_numpy(masters[t]))
        mp.mp_cast_to_16(model.master[t].data_ptr(), model.w16[t].data_ptr(), numels[t], dtype)
        if m0:
            model.m[t].copy_(torch.from_numpy(m0[t]))
            model.v[t].copy_(torch.from_numpy(v0[t]))
    t16 = torch.bfloat16 if dtype == mp.MP_BF16 else torch.float16
    gbufs = [[torch.empty(n, dtype=t16, device="cuda") for n in numels] for _ in range(k)]
    sets = [model.gradset(g) for g in gbufs]
    cfg = mp.scaler_cfg(**scaler) if scaler else mp.scaler_cfg(init_scale=1.0, enabled=False)
    st = mp.mp_state_create(cfg)
    hp = mp.adamw_hparams(**HP)
    reports = []
    try:
        for s in range(steps):
            for i in range(k):
                for t in range(len(numels)):
                    gbufs[i][t].view(torch.int16).copy_(
                        torch.from_numpy(grads[s][i][t].view(np.int16)))
            w = mp.mp_token_weights(counts)
            wo = oracle.token_weights(counts)
            for i in range(k - 1):
                mp.mp_accumulate(model.plan, sets[i], w[i], i == 0)
                orc.accumulate(grads[s][i], wo[i], i == 0)
            lif = k == 1
            mp.mp_unscale_check_norm(model.plan, st, sets[-1], w[-1], lif, max_norm)
            mp.mp_adamw_step(model.plan, st, sets[-1], w[-1], lif, hp)
            mp.mp_scaler_update(st)
            orc.unscale_check_norm(grads[s][-1], wo[-1], lif, max_norm)
            orc.adamw_step(grads[s][-1], wo[-1], lif, **HP)
            orc.scaler_update()
            stt = mp.read_stats(st)
            assert stt["found_inf"] == int(orc.found_inf)
            assert stt["scale"] == orc.scaler.scale and stt["step"] == orc.clock.t
            if not orc.found_inf:
                assert np.float32(stt["grad_norm"]) == np.float32(orc.norm)
            for t in range(len(numels)):
                for name, ref in (("master", orc.masters), ("m", orc.m), ("v", orc.v)):
                    got = getattr(model, name)[t].cpu().numpy()
                    assert np.array_equal(got.view(np.uint32), ref[t].view(np.uint32)), (s, name, t)
                got16 = model.w16[t].cpu().view(torch.int16).numpy().view(np.uint16)
                assert np.array_equal(got16, orc.w16[t]), (s, "w16", t)
            reports.append((stt["found_inf"], stt["grad_norm"], stt["scale"]))
    finally:
        for g in sets:
            mp.mp_gradset_destroy(g)
        mp.mp_state_destroy(st)
        model.close()
    return reports


def bf16_bits(x):
    return oracle.rd16(np.asarray(x, np.float32), oracle.BF16)


def test_huge_finite_gradients(mp):
    """bf16 gradients near the top of fp32's range.  Token weights sum to 1, so the fp32
    accumulation is a convex combination and stays finite; the binary64 sum of squares is
    finite too (no overflow flag), but its square root exceeds fp32: grad_norm = inf, the clip
    coefficient max_norm/(inf + 1e-6) = 0, and the step applies a zero gradient (decay only).
    Without clipping the squares overflow inside AdamW (v = inf, u = 0).  Both sides agree."""
    masters = [np.full(37, 0.5, np.float32)]
    big = bf16_bits(np.full(37, 3.0e38))
    grads = [[[big], [big], [big]]] * 2
    rep = run_both(mp, mp.MP_BF16, masters, grads, counts=[500, 500, 500], steps=2)
    assert rep[0][0] == 0 and rep[0][1] == float("inf")
    run_both(mp, mp.MP_BF16, masters, grads, counts=[500, 500, 500], steps=2, max_norm=0.0)


def test_subnormal_gradients_and_moments(mp):
    """Gradients, weighted products, moments and squares deep in fp32's subnormal range: the
    device keeps denormals exactly like the oracle (no flush to zero)."""
    rng = np.random.default_rng(5)
    n = 4099
    masters = [rng.normal(0, 1e-38, n).astype(np.float32)]
    tiny = np.ldexp(rng.uniform(1, 2, n), rng.integers(-140, -125, n)).astype(np.float32)
    tiny *= np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    g = [bf16_bits(tiny), bf16_bits(tiny * np.float32(0.75))]
    grads = [[[g[0]], [g[1]]], [[g[1]], [g[0]]]]
    m0 = [np.ldexp(np.ones(n), -130).astype(np.float32)]
    v0 = [np.ldexp(np.ones(n), -145).astype(np.float32)]
    run_both(mp, mp.MP_BF16, masters, grads, counts=[401, 509], steps=2, m0=m0, v0=v0)


def test_zero_gradients_decay_only(mp):
    """All-zero gradients: norm 0, no clipping, the step still decays and advances t."""
    masters = [np.linspace(-1, 1, 2049).astype(np.float32), np.ones(5, np.float32)]
    z = [np.zeros(2049, np.uint16), np.zeros(5, np.uint16)]
    grads = [[z, z]] * 2
    rep = run_both(mp, mp.MP_BF16, masters, grads, counts=[400, 400], steps=2)
    assert rep[0] == (0, 0.0, 1.0)


def test_nan_gradient_skips(mp):
    masters = [np.full(3000, 0.25, np.float32)]
    g = bf16_bits(np.full(3000, 1e-3))
    bad = g.copy()
    bad[2999] = 0x7FC1                         # a bf16 NaN in the last element
    grads = [[[g], [bad]], [[g], [g]]]
    rep = run_both(mp, mp.MP_BF16, masters, grads, counts=[450, 460], steps=2)
    assert rep[0][0] == 1 and rep[1][0] == 0


def test_fp16_extremes_with_scaler(mp):
    """fp16 gradients at the largest finite value and the smallest subnormal, k = 1, dynamic
    scale: finite steps update, an fp16 infinity skips and halves S."""
    n = 1025
    masters = [np.full(n, 0.125, np.float32)]
    ext = np.zeros(n, np.uint16)
    ext[0::4], ext[1::4], ext[2::4], ext[3::4] = 0x7BFF, 0x0001, 0xFBFF, 0x8001
    inf = ext.copy()
    inf[7] = 0x7C00
    grads = [[[ext]], [[inf]], [[ext]]]
    sc = dict(init_scale=2.0 ** 4, growth=2.0, backoff=0.5, min_scale=1.0, max_scale=2.0 ** 24,
              interval=2)
    rep = run_both(mp, mp.MP_FP16, masters, grads, counts=[100], steps=3, scaler=sc)
    assert [r[0] for r in rep] == [0, 1, 0] and [r[2] for r in rep] == [16.0, 8.0, 8.0]



def test_no_writes_outside_the_tensors(mp):
    """Ragged tensors laid out with 64-element guard gaps that hold a canary pattern: after
    accumulation, the norm, AdamW, the scaler and the FP8 block cast, every guard is intact
    (no ragged tail writes past its tensor) and every element inside a tensor was written."""
    import torch
    from inputs import configs
    w = configs.make("ragged-4096-small")
    numels = w.numels[:600] + [1, 2, 3, 5, 16, 2047, 2049, 4096, 4097]
    gap = 64
    offs, total = [], 0
    for n in numels:
        offs.append(total)
        total += (n + 15) // 16 * 16 + gap          # 16-element starts: FP8 codes need 16 B
    canary32 = 0x7FA5A5A5                           # a NaN payload no kernel writes
    canary16 = 0x7FA5

    def buf32():
        return torch.full((total,), canary32, dtype=torch.int32, device="cuda").view(torch.float32)

    def buf16():
        return torch.full((total,), canary16, dtype=torch.int16, device="cuda").view(torch.bfloat16)

    bufs = {k: buf32() for k in ("acc", "master", "m", "v")}
    w16 = buf16()
    grads = [buf16() for _ in range(2)]

    def views(b):
        return [b[o:o + n] for o, n in zip(offs, numels)]

    for name in ("master", "m", "v"):
        for x in views(bufs[name]):
            x.fill_(0.25 if name == "master" else 0.0)
    for g in grads:
        for x in views(g):
            x.fill_(1e-3)
    plan = mp.mp_plan_create(numels, mp.MP_BF16, views(bufs["acc"]), views(bufs["master"]),
                             views(bufs["m"]), views(bufs["v"]), views(w16))
    sets = [mp.mp_gradset_create(plan, views(g)) for g in grads]
    st = mp.mp_state_create(mp.scaler_cfg(init_scale=1.0, enabled=False))
    codes = torch.full((total,), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((total // 16 + 64,), canary32, dtype=torch.int32,
                        device="cuda").view(torch.float32)
    try:
        for _ in range(2):
            mp.mp_accumulate(plan, sets[0], 0.5, 1)
            mp.mp_unscale_check_norm(plan, st, sets[1], 0.5, 0, 1.0)
            mp.mp_adamw_step(plan, st, sets[1], 0.5, 0, mp.adamw_hparams())
            mp.mp_scaler_update(st)
        cast = [(o, n) for o, n in zip(offs, numels) if n % 16 == 0]
        assert len(cast) >= 3
        for o, n in cast:
            mp.mp_cast_fp8_blocks(bufs["master"][o:].data_ptr(), codes[o:].data_ptr(),
                                  scales[o // 16:].data_ptr(), n, 16)
        torch.cuda.synchronize()
        inside = np.zeros(total, bool)
        for o, n in zip(offs, numels):
            inside[o:o + n] = True
        for name, b in bufs.items():
            got = b.view(torch.int32).cpu().numpy()
            assert (got[~inside] == canary32).all(), name
            assert (got[inside] != canary32).all(), name
        got16 = w16.view(torch.int16).cpu().numpy()
        assert (got16[~inside] == canary16).all() and (got16[inside] != canary16).all()
        for g in grads:                                   # gradients are read, never written
            assert (g.view(torch.int16).cpu().numpy()[~inside] == canary16).all()
        cast_in = np.zeros(total, bool)
        sc_in = np.zeros(scales.numel(), bool)
        for o, n in cast:
            cast_in[o:o + n] = True
            sc_in[o // 16:o // 16 + n // 16] = True
        assert (codes.cpu().numpy()[~cast_in] == 0x5A).all()
        got_sc = scales.view(torch.int32).cpu().numpy()
        assert (got_sc[~sc_in] == canary32).all() and (got_sc[sc_in] != canary32).all()
        stats = mp.read_stats(st)
        assert stats["found_inf"] == 0 and stats["skipped_total"] == 0
    finally:
        for g in sets:
            mp.mp_gradset_destroy(g)
        mp.mp_state_destroy(st)
        mp.mp_plan_destroy(plan)
