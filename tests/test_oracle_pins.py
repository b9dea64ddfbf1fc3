"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it follows.  None of them re-types the oracle's
formula: they check printed worked examples (tests/golden/), closed forms,
special cases that reduce to library routines, or brute force on tiny inputs.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import BF16, FP16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32bits(x):
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def bits_f32(b):
    return float(np.array([b], dtype=np.uint32).view(np.float32)[0])


def ulp32(x):
    x = abs(np.float32(x))
    return float(np.spacing(x))


# --- rd16 / widen: worked examples and format facts --------------------------

def test_bf16_worked_example_tie_and_101():
    """Section 3 'A bf16 matmul': 1 + 2^-8 is a tie and goes to the even 1.0; 1.01 -> 1.0078125."""
    g = golden("worked_examples.json")["bf16_matmul_example"]
    h = oracle.rd16(np.array([g["tie_input"], g["input_101"]], np.float32), BF16)
    out = oracle.widen16(h, BF16)
    assert out[0] == g["tie_result"]
    assert out[1] == g["result_101"]
    # the next value above 1 in bf16 is 1 + 2^-7 (spacing near 1 is 2^-7)
    f = golden("worked_examples.json")["format_facts"]
    nxt = oracle.widen16(np.array([h[0] + 1], np.uint16), BF16)[0]
    assert nxt - 1.0 == 2.0 ** f["bf16_spacing_near_1_log2"]


def test_fp16_range_facts():
    """Section 2 'Two 16-bit formats': fp16 max 65504, min normal 2^-14, min subnormal 2^-24."""
    f = golden("worked_examples.json")["format_facts"]
    mx = f["fp16_max_finite"]
    vals = np.array([mx, 2.0 ** f["fp16_min_normal_log2"], 2.0 ** f["fp16_min_subnormal_log2"]],
                    np.float32)
    h = oracle.rd16(vals, FP16)
    assert list(h) == [0x7BFF, 0x0400, 0x0001]
    assert list(oracle.widen16(h, FP16)) == list(vals)
    # everything below 65520 (half a spacing above the maximum) stays finite; 65520 overflows
    below = np.nextafter(np.float32(65520.0), np.float32(0))
    h2 = oracle.rd16(np.array([below, 65520.0, 1e6, -65520.0], np.float32), FP16)
    assert list(h2) == [0x7BFF, 0x7C00, 0x7C00, 0xFC00]
    # half the smallest subnormal is a tie and goes to the even value 0; just above it goes to 2^-24
    tiny = np.array([2.0 ** -25, np.nextafter(np.float32(2.0 ** -25), np.float32(1)), -2.0 ** -26],
                    np.float32)
    assert list(oracle.rd16(tiny, FP16)) == [0x0000, 0x0001, 0x8000]


def test_precision_bits():
    """Section 2: p = 8 (bf16) and 11 (fp16): 1 + 2^(1-p) is the next value above 1."""
    f = golden("worked_examples.json")["format_facts"]
    for dt, p in ((BF16, f["bf16_precision_bits"]), (FP16, f["fp16_precision_bits"])):
        one = np.float32(1.0)
        up = np.float32(1.0 + 2.0 ** (1 - p))
        half = np.float32(1.0 + 2.0 ** (-p))           # a tie: goes to the even 1.0
        more = np.float32(1.0 + 2.0 ** (-p) + 2.0 ** (-p - 3))
        out = oracle.widen16(oracle.rd16(np.array([one, up, half, more], np.float32), dt), dt)
        assert list(out) == [1.0, float(up), 1.0, float(up)]


def _fp16_library(x):
    with np.errstate(over="ignore", invalid="ignore"):
        return x.astype(np.float16).view(np.uint16)


def _bf16_library(x):
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _compare_rd16(x, dtype, library, L):
    mine = oracle.rd16(x, dtype, L)
    ref = library(x)
    nan = np.isnan(x)
    bad = (mine != ref) & ~nan
    exp_mask = 0x7F80 if dtype == BF16 else 0x7C00
    man_mask = 0x007F if dtype == BF16 else 0x03FF
    mine_nan = ((mine & exp_mask) == exp_mask) & ((mine & man_mask) != 0)
    return int(bad.sum()), int((nan & ~mine_nan).sum())


# Low halves that sit on or around every rounding position of both formats
# (bf16 rounds at bit 16, normal fp16 at bit 13), plus seeded random ones.
_LOWS = [0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2FFF, 0x3000, 0x3001,
         0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xC000, 0xFFFF]


def _structured_patterns():
    """Every one of the 2^16 high halves (sign, exponent, top mantissa bits) with each low half."""
    rng = np.random.default_rng(20261202)
    lows = np.array(_LOWS + list(rng.integers(0, 1 << 16, 16)), np.uint32)
    high = np.arange(1 << 16, dtype=np.uint32) << 16
    return (high[:, None] | lows[None, :]).ravel().view(np.float32)


def _exhaustive_rd16(dtype, library, L):
    """All 2^32 fp32 patterns: the oracle equals the library conversion (NaN: class only)."""
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 24

    def run(c):
        bits = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64).astype(np.uint32)
        return _compare_rd16(bits.view(np.float32), dtype, library, L)

    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(run, range((1 << 32) // chunk)))
    assert sum(r[0] for r in res) == 0
    assert sum(r[1] for r in res) == 0


def test_rd16_fp16_vs_numpy(orc):
    """Special case reducing to a library routine: numpy's IEEE float32->float16 (RNE), on every
    sign/exponent/top-mantissa prefix with the rounding-relevant tails."""
    assert _compare_rd16(_structured_patterns(), FP16, _fp16_library, orc) == (0, 0)


def test_rd16_bf16_vs_torch(orc):
    """Special case reducing to a library routine: torch's CPU float32->bfloat16 (RNE)."""
    assert _compare_rd16(_structured_patterns(), BF16, _bf16_library, orc) == (0, 0)


FULL = pytest.mark.skipif(os.environ.get("MPSTEP_EXHAUSTIVE") != "1",
                          reason="all 2^32 inputs take ~2 min; set MPSTEP_EXHAUSTIVE=1")


@FULL
def test_rd16_fp16_exhaustive_vs_numpy(orc):
    _exhaustive_rd16(FP16, _fp16_library, orc)


@FULL
def test_rd16_bf16_exhaustive_vs_torch(orc):
    _exhaustive_rd16(BF16, _bf16_library, orc)


def test_widen_exhaustive_both_formats():
    """All 2^16 patterns: the exact fp32 value equals numpy's float16->float32 and bf16<<16."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f16 = oracle.widen16(h, FP16)
    ref16 = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref16)
    assert np.array_equal(f16.view(np.uint32)[~nan], ref16.view(np.uint32)[~nan])
    assert np.isnan(f16[nan]).all()
    b16 = oracle.widen16(h, BF16)
    refb = (h.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(b16.view(np.uint32), refb.view(np.uint32))


def test_rd16_widen_roundtrip_identity():
    """rd16(widen(h)) == h for every non-NaN 16-bit value (every 16-bit value is an fp32 value)."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dt in (BF16, FP16):
        x = oracle.widen16(h, dt)
        back = oracle.rd16(x, dt)
        ok = ~np.isnan(x)
        assert np.array_equal(back[ok], h[ok])


# --- token weights and accumulation -----------------------------------------

def test_token_share_example_seven_thirds():
    """Rust chapter, opening example: counts 2 and 4 with means 1 and 3 give 14/6 = 7/3, not 2."""
    g = golden("rust_chapter_fixtures.json")["token_share_example"]
    w = oracle.token_weights(g["counts"])
    grads = oracle.rd16(np.array(g["mean_losses"], np.float32), BF16)  # 1 and 3 are exact
    acc = np.zeros(1, np.float32)
    oracle.accumulate_tensor(grads[0:1].copy(), acc, BF16, w[0], True)
    oracle.accumulate_tensor(grads[1:2].copy(), acc, BF16, w[1], False)
    num, den = (int(s) for s in g["combined_mean"].split("/"))
    exact = num / den
    assert abs(acc[0] - exact) <= 2 * ulp32(exact)
    assert abs(acc[0] - g["equal_weight_mean"]) > 0.3


def test_backward_seed_shares():
    """Rust chapter: with S = 128, shares 6/9 and 3/9 give f64 seeds 85.333.. and 42.666..;
    the fp32 token weight is the fp32 rounding of that share."""
    g = golden("rust_chapter_fixtures.json")["backward_seeds"]
    w = oracle.token_weights(g["counts"])
    for wi, n, seed in zip(w, g["counts"], g["seeds_f64"]):
        assert g["scale"] * (n / g["total"]) == seed
        assert np.float32(seed / g["scale"]) == wi


def test_token_weight_refusals():
    """Rust chapter 'Extend the existing update...': every micro-batch has targets; N <= 2^53."""
    lim = golden("rust_chapter_fixtures.json")["valid_target_total_limit"]["max_total_log2"]
    with pytest.raises(ValueError):
        oracle.token_weights([3, 0, 2])
    with pytest.raises(ValueError):
        oracle.token_weights([5, -1])
    with pytest.raises(ValueError):
        oracle.token_weights([2 ** lim, 1])
    w = oracle.token_weights([2 ** lim - 1, 1])
    assert w[1] == np.float32(2.0 ** -lim)


def test_hand_example_accumulation():
    """Section 3 'Accumulation': micro-batches of rows [1] and [2,3,4] weighted 1/4 and 3/4 give
    -15; weighting 1/2 gives -10.67 and no weighting -21.3."""
    g = golden("worked_examples.json")["accumulation_example"]
    x = np.array(g["x"], float)
    w0 = g["w"]
    grads = []
    for rows in g["microbatch_rows"]:
        xr = x[np.array(rows) - 1]
        grads.append(np.mean(2 * (w0 * xr - 2 * xr) * xr))
    assert np.allclose(grads, g["microbatch_grads"])
    full = np.mean(2 * (w0 * x - 2 * x) * x)
    assert full == g["one_batch_grad"]
    counts = [len(r) for r in g["microbatch_rows"]]
    for dt, u in ((FP16, 2.0 ** -11), (BF16, 2.0 ** -8)):
        g16 = oracle.rd16(np.array(grads, np.float32), dt)
        w = oracle.token_weights(counts)
        acc = np.zeros(1, np.float32)
        for i in range(2):
            oracle.accumulate_tensor(g16[i:i + 1].copy(), acc, dt, w[i], i == 0)
        bound = sum(float(wi) * abs(gi) for wi, gi in zip(w, grads)) * u + 4 * ulp32(15.0)
        assert abs(acc[0] - g["one_batch_grad"]) <= bound
        assert abs(acc[0] - g["half_weight_grad"]) > 1.0
        assert abs(acc[0] - g["unweighted_grad"]) > 1.0
    # the loss side of the same table: sum_i (n_i/N) L_i = 7.5
    L = [1.0, 29.0 / 3.0]
    assert abs(sum(n / 4 * li for n, li in zip(counts, L)) - g["one_batch_loss"]) < 1e-12


def test_micro_batches_equal_one_big_batch():
    """Section 4 catalogue: micro-batches of 5, 11 and 16 rows equal one batch of 32 (up to the
    16-bit rounding of each micro-batch gradient and fp32 accumulation)."""
    g = golden("worked_examples.json")["micro_batches_equal_one_batch"]
    rng = np.random.default_rng(7)
    n_params = 257
    per_row = rng.normal(0, 1e-2, size=(g["total_rows"], n_params))
    full = per_row.mean(axis=0)
    bounds = np.cumsum([0] + g["rows"])
    mb = [per_row[a:b].mean(axis=0) for a, b in zip(bounds[:-1], bounds[1:])]
    w = oracle.token_weights(g["rows"])
    for dt, u in ((FP16, 2.0 ** -11), (BF16, 2.0 ** -8)):
        acc = np.zeros(n_params, np.float32)
        for i, gi in enumerate(mb):
            oracle.accumulate_tensor(oracle.rd16(gi.astype(np.float32), dt), acc, dt, w[i], i == 0)
        bound = sum(float(wi) * np.abs(gi) for wi, gi in zip(w, mb)) * (u + 4 * 2.0 ** -24)
        bound += 4 * 2.0 ** -24 * np.abs(full)
        assert np.all(np.abs(acc - full) <= bound)
        # equal weights 1/3 give a different gradient whenever the sizes differ
        eq = sum(m / 3 for m in mb)
        assert np.max(np.abs(acc - eq)) > 10 * np.max(bound)


def test_first_overwrites_dropped_gradients():
    """Section 2 'Dynamic scaling' and pitfall 13: after a skip the bad gradient is dropped;
    the next update's first micro-batch overwrites the buffer."""
    acc = np.array([np.inf, np.nan, -np.inf, 5.0], np.float32)
    g16 = oracle.rd16(np.array([1.0, -2.0, 0.5, 0.0], np.float32), BF16)
    oracle.accumulate_tensor(g16, acc, BF16, np.float32(0.25), True)
    assert list(acc) == [0.25, -0.5, 0.125, 0.0]


# --- unscale, overflow, norm, clip -------------------------------------------

def test_fp16_underflow_rescued_by_scaling():
    """Section 2 'Loss scaling' (and the Key Takeaways): fp16 gradients below 2^-24 flush to zero;
    with S = 2^16 they survive and unscaling recovers them to fp16 precision."""
    octaves = np.arange(-30, -20)
    mant = np.linspace(1.0, 2.0, 64, endpoint=False)[1:]
    g_true = np.concatenate([np.ldexp(mant, int(e)) for e in octaves]).astype(np.float32)
    # S = 1: everything at or below 2^-25 becomes exactly zero
    h1 = oracle.rd16(g_true, FP16)
    back1 = oracle.widen16(h1, FP16)
    assert np.all(back1[g_true <= 2.0 ** -25] == 0.0)
    assert np.all(back1[g_true > 2.0 ** -25] > 0.0)
    # exactly half of the ten octaves [2^-30, 2^-20) flush
    assert np.count_nonzero(back1 == 0) == g_true.size // 2
    # S = 2^16: nothing flushes; unscaled through the oracle the relative error is <= 2^-11
    S = np.float32(2.0 ** 16)
    hS = oracle.rd16(g_true * S, FP16)
    for j in range(g_true.size):
        fi, ss = oracle.unscale_sumsq_tensor(None, hS[j:j + 1].copy(), 1, FP16, 1.0, 1,
                                             oracle.unscale_factor(S))
        assert not fi
        g = math.sqrt(ss)
        assert abs(g - g_true[j]) <= 2.0 ** -11 * g_true[j]


def test_loss_scaler_hand_trace():
    """Section 3 'Loss scaling' table: S = 8, growth 2, backoff 1/2, interval 2, SGD lr 0.5."""
    g = golden("worked_examples.json")["loss_scaler_trace"]
    sc = oracle.make_scaler(init_scale=g["init_scale"], growth=g["growth"], backoff=g["backoff"],
                            interval=g["interval"], min_scale=1.0, max_scale=2.0 ** 64)
    w = g["w0"]
    for k, sg in enumerate(g["scaled_g"]):
        val = np.float32(np.inf if sg == "inf" else sg)
        h = oracle.rd16(np.array([val], np.float32), FP16)
        fi, ss = oracle.unscale_sumsq_tensor(None, h, 1, FP16, 1.0, 1,
                                             oracle.unscale_factor(sc.scale))
        assert (not fi) == g["finite"][k]
        if not fi:
            ug = math.sqrt(ss)
            assert ug == g["unscaled_g"][k]
            w = w - g["sgd_lr"] * ug
        oracle.scaler_update(sc, fi)
        assert w == g["w_after"][k]
        assert sc.scale == g["scale_after"][k]
        assert sc.good_steps == g["good_steps_after"][k]
        assert sc.skipped == (0 if g["finite"][k] else 1)


def test_rust_scaler_fixture_growth_and_backoff():
    """Rust chapter: DynamicLossScaler(128, 1, 256, 1): a committed update grows 128 -> 256; the
    late-overflow probe backs off 128 -> 64; growth stops at the maximum."""
    g = golden("rust_chapter_fixtures.json")["scaler_fixture"]
    sc = oracle.make_scaler(init_scale=g["init_scale"], min_scale=g["min_scale"],
                            max_scale=g["max_scale"], interval=g["interval"])
    oracle.scaler_update(sc, False)
    assert sc.scale == g["after_commit"]
    oracle.scaler_update(sc, False)
    assert sc.scale == g["max_scale"]
    sc2 = oracle.make_scaler(init_scale=g["init_scale"], min_scale=g["min_scale"],
                             max_scale=g["max_scale"], interval=g["interval"])
    oracle.scaler_update(sc2, True)
    assert sc2.scale == g["after_overflow"] and sc2.good_steps == 0
    for _ in range(10):
        oracle.scaler_update(sc2, True)
    assert sc2.scale == g["min_scale"]


def test_scaler_disabled_keeps_scale():
    """bf16 needs no scaler (section 2 'Dynamic scaling', last sentence): S stays fixed, but the
    skip is still reported."""
    sc = oracle.make_scaler(init_scale=8.0, enabled=False, interval=1, min_scale=1.0)
    oracle.scaler_update(sc, True)
    assert sc.scale == 8.0 and sc.skipped == 1
    oracle.scaler_update(sc, False)
    assert sc.scale == 8.0 and sc.skipped == 0 and sc.skipped_total == 1


def test_unscale_before_clip():
    """Section 4 catalogue: clip to 1 of a gradient of norm 5 scaled by 1024: the norm is taken in
    true units (5), so the coefficient is about 1/5, not 1/5120."""
    g = golden("worked_examples.json")["unscale_before_clip"]
    S = np.float32(g["scale"])
    h = oracle.rd16(np.array(g["grad"], np.float32) * S, FP16)
    fi, ss = oracle.unscale_sumsq_tensor(None, h, 2, FP16, 1.0, 1, oracle.unscale_factor(S))
    norm, coef = oracle.norm_and_coef(ss, fi, g["clip"])
    assert norm == g["true_norm"]
    assert abs(coef - 1.0 / g["true_norm"]) < 1e-6
    clipped = np.array(g["grad"]) * coef
    assert abs(np.linalg.norm(clipped) - g["clip"]) < 1e-6


def test_clip_only_above_limit():
    """Rust chapter fixtures: norm 0.93899.. under a limit of 1 is not clipped; 1.48536.. is
    clipped to 1."""
    g = golden("rust_chapter_fixtures.json")["clip_fixtures"]
    for nrm, clipped in ((g["unclipped_norm"], False), (g["clipped_norm"], True)):
        x = np.float32(nrm)
        norm, coef = oracle.norm_and_coef(float(x) ** 2, False, g["max_norm"])
        assert norm == x
        if clipped:
            assert abs(norm * coef - g["max_norm"]) < 1e-6
        else:
            assert coef == 1.0
    # no clipping requested, or an overflowed step: coefficient 1
    assert oracle.norm_and_coef(100.0, False, 0.0)[1] == 1.0
    assert oracle.norm_and_coef(float("inf"), True, 1.0)[1] == 1.0


def test_global_norm_closed_forms():
    """'Megatron Internals III' section 9: global_norm = sqrt(sum_i ||g_i||^2) over all tensors."""
    # a constant c over n elements has norm c*sqrt(n)
    n = 1_000_000
    acc = np.full(n, 0.5, np.float32)
    fi, ss = oracle.unscale_sumsq_tensor(acc, None, n, BF16, 1.0, 0, 1.0)
    assert not fi and ss == 0.25 * n
    assert oracle.norm_and_coef(ss, fi, 0.0)[0] == 500.0
    # a 3-4-5 triangle split across two tensors: the norm spans tensors
    parts = []
    for val in (3.0, 4.0):
        fi, s = oracle.unscale_sumsq_tensor(np.array([val], np.float32), None, 1, BF16, 1.0, 0, 1.0)
        parts.append(s)
    assert oracle.norm_and_coef(oracle.sum_in_order(parts), False, 0.0)[0] == 5.0
    # unscaling by 1/S happens before the squares
    acc = np.array([3.0 * 1024, 4.0 * 1024], np.float32)
    fi, s = oracle.unscale_sumsq_tensor(acc, None, 2, FP16, 1.0, 0, np.float32(1 / 1024))
    assert s == 25.0


def test_step_norm_and_overflow_span_all_tensors():
    """'Megatron Internals III' sections 6 and 9: the overflow decision and the norm cover every
    tensor of the update, not one of them."""
    masters = [np.zeros(1, np.float32), np.zeros(1, np.float32), np.zeros(2, np.float32)]
    st = oracle.OracleStep(BF16, masters, [oracle.rd16(x, BF16) for x in masters])
    g = [oracle.rd16(np.array(v, np.float32), BF16) for v in ([3.0], [4.0], [0.0, 12.0])]
    fi, ss, norm, coef = st.unscale_check_norm(g, 1.0, True, 1.0)
    assert not fi and ss == 169.0 and norm == 13.0
    assert abs(coef - 1 / 13) < 1e-7
    for t in range(3):
        bad = [x.copy() for x in g]
        bad[t][0] = 0x7F80
        assert st.unscale_check_norm(bad, 1.0, True, 1.0)[0]


def test_sumsq_exact_brute_force():
    """Brute force: the compensated binary64 sum equals the exact rational sum of squares to
    within a couple of binary64 roundings, for sizes and magnitudes far apart."""
    rng = np.random.default_rng(3)
    for n in (1, 7, 1000, 20000):
        acc = (rng.standard_normal(n) * np.exp(rng.uniform(-20, 20, n))).astype(np.float32)
        fi, s = oracle.unscale_sumsq_tensor(acc, None, n, BF16, 1.0, 0, 1.0)
        exact = sum(Fraction(float(a)) ** 2 for a in acc)
        assert abs(Fraction(s) - exact) <= exact * Fraction(2, 2 ** 52)


def test_overflow_flag_any_tensor_any_value():
    """Section 2 'Dynamic scaling': one non-finite entry anywhere poisons the step."""
    for bad in (np.inf, -np.inf, np.nan):
        acc = np.zeros(1000, np.float32)
        acc[617] = bad
        fi, _ = oracle.unscale_sumsq_tensor(acc, None, 1000, FP16, 1.0, 0, 1.0)
        assert fi
    # a finite fp16 gradient that is huge stays finite after unscaling
    h = np.array([0x7BFF], np.uint16)
    fi, _ = oracle.unscale_sumsq_tensor(None, h, 1, FP16, 1.0, 1, np.float32(2.0 ** -16))
    assert not fi


# --- AdamW ---------------------------------------------------------------------

def _adam_run(g_steps, w0=0.5, lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.0, dtype=BF16,
              clip=0.0, S=1.0):
    masters = [np.array([w0], np.float32)]
    w16 = [oracle.rd16(masters[0], dtype)]
    sc = oracle.make_scaler(init_scale=S, enabled=False)
    st = oracle.OracleStep(dtype, masters, w16, scaler=sc)
    for g in g_steps:
        h = [oracle.rd16(np.array([g * S], np.float32), dtype)]
        st.unscale_check_norm(h, 1.0, True, clip)
        st.adamw_step(h, 1.0, True, lr, b1, b2, eps, wd)
        st.scaler_update()
    return st


def test_adamw_first_step_closed_form():
    """With m0 = v0 = 0 the first bias-corrected step is u = g/(|g| + eps) (the update in words on
    'Your weights fit on one device...'), and decoupled decay adds lr*lambda*w0."""
    lr, wd, eps = 3e-4, 0.1, 1e-8
    for g in (1.0, -0.25, 3e-3, -7e-5, 1e-9, 0.0):
        gq = float(oracle.widen16(oracle.rd16(np.array([g], np.float32), BF16), BF16)[0])
        w0 = 0.75
        st = _adam_run([g], w0=w0, lr=lr, wd=wd, eps=eps)
        u = gq / (abs(gq) + eps)
        w1 = w0 - lr * (u + wd * w0)
        assert abs(st.masters[0][0] - w1) <= 4 * ulp32(w1)
        ob1, ob2 = 1 - float(np.float32(0.9)), 1 - float(np.float32(0.95))
        assert abs(st.m[0][0] - ob1 * gq) <= ulp32(ob1 * gq) + 1e-45
        assert abs(st.v[0][0] - ob2 * gq * gq) <= 2 * ulp32(ob2 * gq * gq) + 1e-45
        assert st.clock.t == 1
        assert st.w16[0][0] == oracle.rd16(st.masters[0], BF16)[0]


def test_adamw_moments_hold_unscaled_gradients():
    """'Megatron Internals III' section 8 and section 9 steps 3-6: the optimizer sees unscaled fp32
    gradients, so with S = 2^10 the first moments are (1-b1) g and (1-b2) g^2 in true units."""
    ob1, ob2 = 1 - float(np.float32(0.9)), 1 - float(np.float32(0.95))
    for S in (1.0, 2.0 ** 10, 2.0 ** 16):
        st = _adam_run([0.375], w0=0.5, dtype=FP16, S=S)
        assert abs(st.m[0][0] - ob1 * 0.375) <= ulp32(ob1 * 0.375)
        assert abs(st.v[0][0] - ob2 * 0.375 ** 2) <= 2 * ulp32(ob2 * 0.375 ** 2)


def test_adamw_zero_gradient_still_decays():
    """Rust chapter 'Discard a failed partial logical update': an AdamW step with zero gradients
    can still apply weight decay and advance the optimizer state."""
    st = _adam_run([0.0], w0=2.0, lr=0.01, wd=0.5)
    assert abs(st.masters[0][0] - 2.0 * (1 - 0.01 * 0.5)) <= 2 * ulp32(2.0)
    assert st.clock.t == 1 and st.m[0][0] == 0 and st.v[0][0] == 0


def test_adamw_scale_invariant_first_step():
    """Adam's first step is invariant to a positive rescaling of the gradient (|g| >> eps), so the
    clip coefficient does not change it -- but it is applied (m scales by the coefficient)."""
    st1 = _adam_run([4.0], clip=0.0)
    st2 = _adam_run([4.0], clip=0.5)
    assert abs(st1.masters[0][0] - st2.masters[0][0]) <= 2 * ulp32(st1.masters[0][0])
    ob1 = 1 - float(np.float32(0.9))
    assert abs(st2.m[0][0] - ob1 * 4.0 * (0.5 / (4.0 + 1e-6))) <= 2 * ulp32(st2.m[0][0])


def test_adamw_second_step_bias_correction_closed_form():
    """Two steps with gradients g1, g2: m2 = (1-b1)(b1 g1 + g2), v2 = (1-b2)(b2 g1^2 + g2^2),
    bias corrections 1 - b^2; w2 = w1 - lr (m2/(1-b1^2)) / (sqrt(v2/(1-b2^2)) + eps)."""
    b1, b2, lr, eps = 0.9, 0.95, 1e-2, 1e-8
    for g1, g2 in ((0.5, -0.25), (1.0, 1.0), (-0.125, 2.0)):
        st = _adam_run([g1, g2], w0=1.0, lr=lr, b1=b1, b2=b2, eps=eps)
        B1, B2 = float(np.float32(b1)), float(np.float32(b2))
        u1 = g1 / (abs(g1) + eps)
        w1 = 1.0 - lr * u1
        m2 = (1 - B1) * (B1 * g1 + g2)
        v2 = (1 - B2) * (B2 * g1 * g1 + g2 * g2)
        u2 = (m2 / (1 - B1 ** 2)) / (math.sqrt(v2 / (1 - B2 ** 2)) + eps)
        w2 = w1 - lr * u2
        assert abs(st.masters[0][0] - w2) <= 8 * ulp32(w2)
        assert st.clock.t == 2


def test_adamw_constant_gradient_trajectory():
    """A constant gradient makes the bias-corrected moments g and g^2 at every step, so each step
    moves w by lr (no decay): after t steps w = w0 - t*lr."""
    t, lr = 25, 1e-3
    st = _adam_run([0.5] * t, w0=1.0, lr=lr)
    assert abs(st.masters[0][0] - (1.0 - t * lr)) <= 4 * t * ulp32(1.0)
    assert st.v[0][0] >= 0


def _bf16_values(xs):
    """The values as bf16 numbers (what the oracle sees after the 16-bit cast)."""
    return [float(y) for y in oracle.widen16(oracle.rd16(np.asarray(xs, np.float32), BF16), BF16)]


def test_adamw_moments_track_exact_moving_averages():
    """lr = 0 freezes the weights, so only the moment recursion acts ('Your weights fit on one
    device...': m and v are running averages of g and g^2 with decay beta).  Over 50 steps of
    gradients that vary in sign and size, m and v stay within a rigorous fp32 rounding bound of
    the exact averages m_t = b1 m_(t-1) + (1-b1) g_t and v_t = b2 v_(t-1) + (1-b2) g_t^2 (b the
    fp32 betas, 1-b exact by Sterbenz), and the clock holds t = 50 and b^50 to binary64 accuracy."""
    rng = np.random.default_rng(5)
    gs = _bf16_values(rng.normal(0, 1, 50) * np.exp(rng.uniform(-6, 2, 50)))
    st = _adam_run(gs, w0=0.5, lr=0.0)
    assert st.masters[0][0] == np.float32(0.5)
    u = 2.0 ** -24
    for beta, got, sq in ((float(np.float32(0.9)), st.m[0][0], False),
                          (float(np.float32(0.95)), st.v[0][0], True)):
        exact, bound = 0.0, 0.0
        for g in gs:
            term = (1 - beta) * (g * g if sq else g)    # g*g is exact: bf16 has 8 bits
            prev = exact
            exact = beta * prev + term
            # three roundings per step (product, product, sum), plus the carried error
            bound = beta * bound + u * (abs(beta * prev) + abs(term) + abs(exact)) + 1e-45
        assert abs(float(got) - exact) <= bound, (got, exact, bound)
    assert st.clock.t == 50
    for p, beta in ((st.clock.p1, float(np.float32(0.9))), (st.clock.p2, float(np.float32(0.95)))):
        assert abs(p - beta ** 50) <= 1e-13 * beta ** 50


def test_adamw_zero_betas_trajectory_with_varying_gradients():
    """With b1 = b2 = 0 the moments are the current gradient and its square and both bias
    corrections are 1, so every step is w <- w - lr (g/(|g| + eps) + lambda w) (decoupled decay,
    'Accumulate gradients and recompute activations').  Thirty steps of gradients that change
    sign and size, including a zero, follow that recursion to within a few fp32 roundings a
    step."""
    rng = np.random.default_rng(6)
    raw = rng.normal(0, 1, 30) * np.exp(rng.uniform(-8, 3, 30))
    raw[7] = 0.0
    gs = _bf16_values(raw)
    lr, wd, eps, w = 1e-2, 0.1, 1e-8, 0.75
    st = _adam_run(gs, w0=w, lr=lr, b1=0.0, b2=0.0, eps=eps, wd=wd)
    for g in gs:
        u = g / (abs(g) + eps)
        w = w - lr * (u + wd * w)
    assert abs(st.masters[0][0] - w) <= 6 * len(gs) * ulp32(w)
    assert st.m[0][0] == np.float32(gs[-1]) and st.v[0][0] == np.float32(gs[-1] ** 2)


def test_master_absorbs_sub_spacing_update():
    """Section 2 'Why the weights stay float32': a weight of 1 updated by 1e-3 rounds back to 1 in
    bf16, but the fp32 master keeps the change; ten such updates move the bf16 copy."""
    st = _adam_run([0.5], w0=1.0, lr=1e-3)
    assert abs(st.masters[0][0] - 0.999) <= 2 * ulp32(0.999)
    assert st.w16[0][0] == 0x3F80            # bf16 1.0
    st = _adam_run([0.5] * 10, w0=1.0, lr=1e-3)
    assert abs(st.masters[0][0] - 0.99) <= 20 * ulp32(0.99)
    assert oracle.widen16(st.w16[0], BF16)[0] == 0.98828125   # nearest bf16 to 0.99


def test_skip_leaves_state_bit_identical():
    """Rust chapter 'Discard a failed partial logical update' and pitfalls 12-13: an overflowed
    step changes no weight, moment, beta power or step count; S backs off."""
    rng = np.random.default_rng(11)
    masters = [rng.normal(0, 0.02, 300).astype(np.float32), rng.normal(0, 0.02, 77).astype(np.float32)]
    w16 = [oracle.rd16(x, FP16) for x in masters]
    st = oracle.OracleStep(FP16, masters, w16, scaler=oracle.make_scaler(init_scale=128.0,
                                                                         interval=1, max_scale=256.0))
    g = [oracle.rd16(rng.normal(0, 1e-3, x.size).astype(np.float32) * 128, FP16) for x in masters]
    st.accumulate(g, 1.0, True)
    st.unscale_check_norm(None, 1.0, False, 1.0)
    assert st.adamw_step() is True
    st.scaler_update()
    assert st.scaler.scale == 256.0
    snap = [a.copy() for a in st.masters + st.m + st.v + st.w16]
    clock = (st.clock.t, st.clock.p1, st.clock.p2)
    g[1][40] = 0x7C00
    st.accumulate(g, 1.0, True)
    fi, *_ = st.unscale_check_norm(None, 1.0, False, 1.0)
    assert fi and st.adamw_step() is False
    st.scaler_update()
    assert all(np.array_equal(a.view(np.uint8), b.view(np.uint8))
               for a, b in zip(snap, st.masters + st.m + st.v + st.w16))
    assert (st.clock.t, st.clock.p1, st.clock.p2) == clock
    assert st.scaler.scale == 128.0 and st.scaler.skipped == 1


def test_fold_last_microbatch_equals_accumulating_it():
    """The last micro-batch folded into the norm and update passes gives the same gradient bits as
    accumulating it first (the same two fp32 operations in the same order)."""
    rng = np.random.default_rng(5)
    sizes = [1000, 3, 4097]
    def fresh():
        masters = [rng.normal(0, 0.02, n).astype(np.float32) for n in sizes]
        return masters
    base = fresh()
    grads = [[oracle.rd16(rng.normal(0, 1e-3, n).astype(np.float32), BF16) for n in sizes]
             for _ in range(3)]
    w = oracle.token_weights([400, 512, 451])
    out = []
    for fold in (False, True):
        masters = [x.copy() for x in base]
        st = oracle.OracleStep(BF16, masters, [oracle.rd16(x, BF16) for x in masters])
        st.accumulate(grads[0], w[0], True)
        st.accumulate(grads[1], w[1], False)
        if fold:
            st.unscale_check_norm(grads[2], w[2], False, 1.0)
            st.adamw_step(grads[2], w[2], False)
        else:
            st.accumulate(grads[2], w[2], False)
            st.unscale_check_norm(None, 1.0, False, 1.0)
            st.adamw_step()
        out.append((st.sumsq, [a.copy() for a in st.masters + st.m + st.v + st.w16]))
    assert out[0][0] == out[1][0]
    assert all(np.array_equal(a, b) for a, b in zip(out[0][1], out[1][1]))


def test_weight_decay_multiplier_zero_means_no_decay():
    """A tensor with decay multiplier 0 (e.g. a norm vector) only gets the Adam update."""
    masters = [np.array([1.0], np.float32), np.array([1.0], np.float32)]
    st = oracle.OracleStep(BF16, masters, [oracle.rd16(x, BF16) for x in masters], wd_mult=[1.0, 0.0])
    g = [oracle.rd16(np.array([0.0], np.float32), BF16)] * 2
    st.unscale_check_norm(g, 1.0, True, 0.0)
    st.adamw_step(g, 1.0, True, lr=0.1, weight_decay=0.5)
    assert st.masters[0][0] == np.float32(1.0) - np.float32(0.1) * np.float32(0.5)
    assert st.masters[1][0] == 1.0


# --- memory accounting ---------------------------------------------------------

def test_sixteen_bytes_per_parameter():
    """Chapter 41 equation (41.1) and 'Megatron Internals III' section 1: 2+2+4+4+4 = 16 B."""
    g = golden("memory_accounting.json")
    assert sum(g["bytes_per_param"]["components"].values()) == g["bytes_per_param"]["total"]
    assert oracle.model_state_bytes(1) == g["bytes_per_param"]["total"]
    ex = g["exercise_41_1"]
    assert oracle.model_state_bytes(ex["params"]) == ex["bytes"]


# --- fine-grained FP8 ('Chapter 41 Training at Scale', section 41.5) -----------------

def test_e4m3_format_facts():
    """E4M3: largest finite 448 (the listing's max_value), smallest normal 2^-6, smallest
    subnormal 2^-9; ties go to even; NaN keeps its sign; no infinity (saturate at 448)."""
    vals = [448.0, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10, 1.0, 1.0625, 1.1875, 3 * 2.0 ** -10,
            -1.5, float("inf"), 1e9, -0.0]
    assert [int(c) for c in oracle.e4m3(vals)] == [0x7E, 0x08, 0x01, 0x00, 0x38, 0x38, 0x3A,
                                                   0x02, 0xBC, 0x7E, 0x7E, 0x80]
    assert oracle.e4m3([float("nan")])[0] & 0x7F == 0x7F
    assert oracle.e4m3_value([0x7E])[0] == 448.0 and np.isnan(oracle.e4m3_value([0x7F])[0])


def test_e4m3_roundtrip_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_value(codes)
    ok = ~np.isnan(vals)
    assert ok.sum() == 254
    back = oracle.e4m3(vals[ok])
    same = back == codes[ok]
    # the two zeros both encode; -0 keeps its sign
    assert same.all()


def test_e4m3_vs_torch_float8():
    """Special case reducing to a library routine: torch's float32 -> float8_e4m3fn (RNE) on every
    sign/exponent/top-mantissa prefix with rounding-relevant tails, below the overflow threshold
    464 (where torch returns NaN and this reading saturates)."""
    import torch
    x = _structured_patterns()
    keep = np.isnan(x) | (np.abs(x) < 464.0)
    x = x[keep]
    mine = oracle.e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = np.isnan(x)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert ((mine[nan] & 0x7F) == 0x7F).all()


def test_fp8_block_cast_follows_the_listing():
    """Listing 41.5: scale = max|x|/max_value per block of 16 (a zero block takes 1); the
    dequantised value x' = e4m3(x/scale) * scale is within half an E4M3 spacing of x."""
    rng = np.random.default_rng(41)
    x = (rng.standard_normal(16 * 64) * np.exp(rng.uniform(-8, 8, 16 * 64))).astype(np.float32)
    x[32:48] = 0.0
    codes, scales = oracle.fp8_block_cast(x, 16)
    blocks = x.reshape(-1, 16)
    want = np.max(np.abs(blocks), axis=1) / np.float32(448.0)
    want = np.where(want == 0, np.float32(1.0), want).astype(np.float32)
    assert np.array_equal(scales, want)
    deq = (oracle.e4m3_value(codes).reshape(-1, 16) * scales[:, None]).astype(np.float32)
    y = np.abs(blocks / scales[:, None])
    bound = np.where(y >= 2.0 ** -6, 2.0 ** -4 * y, 2.0 ** -10) * scales[:, None] * (1 + 1e-6)
    assert (np.abs(deq - blocks) <= bound).all()
    with pytest.raises(ValueError):
        oracle.fp8_block_cast(np.zeros(17, np.float32), 16)


def test_fp8_block_with_nan_follows_the_listing():
    """Listing 41.5 takes the block scale with np.max, which propagates NaN: a block holding one
    NaN gets a NaN scale (written as the quiet NaN 0x7FC00000) and every value of it a NaN code,
    whose sign bit is the value's; a block whose maximum is infinite gets an infinite scale, its
    finite values code to signed zero and inf / inf to NaN with the value's sign."""
    x = np.linspace(-3.0, 3.0, 64).astype(np.float32)
    x[16 + 5] = np.nan                       # block 1: one NaN among finite values of both signs
    x[32 + 2] = np.inf                       # block 2: +inf and -inf, the rest finite
    x[32 + 9] = -np.inf
    x[48:64] = 0.0
    x[48 + 7] = np.nan                       # block 3: NaN among zeros
    codes, scales = oracle.fp8_block_cast(x, 16)
    blocks = x.reshape(-1, 16)
    with np.errstate(invalid="ignore"):
        listing = np.max(np.abs(blocks), axis=-1) / np.float32(448.0)
    listing = np.where(listing == 0, np.float32(1.0), listing).astype(np.float32)
    assert np.array_equal(np.isnan(scales), np.isnan(listing))
    assert np.isnan(scales[[1, 3]]).all()
    assert (scales.view(np.uint32)[[1, 3]] == 0x7FC00000).all()
    fin = ~np.isnan(listing)
    assert np.array_equal(scales[fin], listing[fin])
    assert scales[2] == np.inf
    sign = (x.view(np.uint32) >> 24).astype(np.uint8) & 0x80
    for b in (1, 3):
        c = codes[16 * b:16 * b + 16]
        assert np.array_equal(c, sign[16 * b:16 * b + 16] | 0x7F)
    c2 = codes[32:48]
    assert c2[2] == 0x7F and c2[9] == 0xFF
    rest = np.array([i for i in range(16) if i not in (2, 9)])
    assert np.array_equal(c2[rest], sign[32 + rest])      # finite / inf = signed zero


def test_fp8_block_scales_help_the_small_block():
    """Section 41.5: one scale for a whole tensor forces small blocks onto a coarse step; a scale
    per block keeps their relative precision."""
    big = np.full(16, 1000.0, np.float32)
    small = np.linspace(1e-3, 2e-3, 16).astype(np.float32)
    x = np.concatenate([big, small])
    c_blk, s_blk = oracle.fp8_block_cast(x, 16)
    c_one, s_one = oracle.fp8_block_cast(x, 32)
    d_blk = oracle.e4m3_value(c_blk) * np.repeat(s_blk, 16)
    d_one = oracle.e4m3_value(c_one) * np.repeat(s_one, 32)
    rel_blk = np.abs(d_blk[16:] - small) / small
    rel_one = np.abs(d_one[16:] - small) / small
    assert rel_blk.max() <= 2.0 ** -4
    assert rel_one.max() >= 0.5                       # flushed to (nearly) zero
