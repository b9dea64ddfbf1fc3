"""The C-ABI library on the host, without a GPU (CPU only).

Checks that libmpstep.so loads and exports every entry point include/mpstep.h
declares, and exercises the host-only logic: status strings, token weights,
memory accounting, the chunk table, and argument validation that returns before
any device work.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpstep.h")


@pytest.fixture(scope="module")
def mp():
    import optimizer_step_tensor_amd as m
    m.lib()
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mp_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_function_is_exported(mp):
    names = declared_functions()
    assert len(names) >= 20
    raw = ctypes.CDLL(mp.build.LIB)
    missing = [n for n in names if not hasattr(raw, n)]
    assert missing == []
    assert sorted(mp.ENTRY_POINTS) == names


def test_header_constants_match_the_binding(mp):
    src = open(HEADER).read()
    for name in ("MP_STATE_BLOB_BYTES", "MP_NOALLOC_MAX_NORM_BLOCKS"):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, src)
        assert m and int(m.group(1)) == getattr(mp, name), name


def test_status_strings_and_version(mp):
    assert mp.mp_abi_version() == 1
    assert [mp.mp_status_string(s) for s in range(6)] == [
        "MP_OK", "MP_ERR_INVALID", "MP_ERR_ALIGN", "MP_ERR_NOMEM", "MP_ERR_HIP", "MP_ERR_ORDER"]


def test_token_weights_match_the_oracle(mp):
    rng = np.random.default_rng(1)
    for k in (1, 2, 3, 4, 8, 31):
        counts = rng.integers(1, 10 ** 6, k)
        assert np.array_equal(np.array(mp.mp_token_weights(counts), np.float32),
                              oracle.token_weights(counts))
    with pytest.raises(mp.MpError) as e:
        mp.mp_token_weights([4, 0])
    assert e.value.status == mp.MP_ERR_INVALID
    with pytest.raises(mp.MpError):
        mp.mp_token_weights([2 ** 53, 1])
    with pytest.raises(mp.MpError):
        mp.mp_token_weights([])


def test_bytes_per_parameter(mp):
    """'Chapter 41 Training at Scale' equation (41.1): 16 bytes, plus the fp32 accumulator."""
    for dt in (mp.MP_BF16, mp.MP_FP16):
        assert mp.mp_state_bytes_per_param(dt, False) == oracle.model_state_bytes(1) == 16
        assert mp.mp_state_bytes_per_param(dt, True) == 20


def _check_layout(mp, numel, cus):
    ch, chunks = mp.mp_chunk_layout(numel, cus)
    assert ch % 2048 == 0 and ch & (ch - 1) == 0 and 2048 <= ch <= 65536
    covered = [0] * len(numel)
    prev = (-1, -1)
    for t, s, ln in chunks:
        assert 1 <= ln <= ch
        assert s % ch == 0                      # chunks start on chunk (hence vector) boundaries
        assert s == covered[t]                  # contiguous, in order, no overlap or gap
        assert (t, s) > prev
        prev = (t, s)
        covered[t] = s + ln
    assert covered == list(numel)               # every element exactly once
    return ch, chunks


def test_chunk_layout_covers_every_element_once(mp):
    from inputs import configs
    for name in ("edges", "llama-10.5M", "gpt-124M", "ragged-4096-small", "llama3-8B"):
        w = configs.make(name)
        _check_layout(mp, w.numels, 256)
    rng = np.random.default_rng(9)
    for _ in range(20):
        n = rng.integers(1, 200)
        numel = list(rng.integers(1, 300_000, n))
        _check_layout(mp, numel, int(rng.integers(1, 400)))


def test_chunk_count_at_full_size(mp):
    """The 8B-parameter list: one chunk per 2048 elements of every tensor, ragged tails counted."""
    import ctypes as C
    from inputs import configs
    numel = configs.make("llama3-8B").numels
    ne = (C.c_int64 * len(numel))(*numel)
    ch, nc = C.c_int32(), C.c_int64()
    assert mp.lib().mp_chunk_layout(len(numel), ne, 256, C.byref(ch), C.byref(nc), None, None,
                                    None, 0) == 0
    assert nc.value == sum(-(-n // ch.value) for n in numel)
    assert ch.value == 2048


def test_validation_before_any_device_work(mp):
    """Refusals that return before the library touches a device."""
    L = mp.lib()
    out = ctypes.c_void_p()
    ne = (ctypes.c_int64 * 1)(16)
    good = (ctypes.c_void_p * 1)(0x10000)
    bad = (ctypes.c_void_p * 1)(0x10008)           # 8-byte aligned only
    PP = ctypes.POINTER(ctypes.c_void_p)
    g = ctypes.cast(good, PP)
    assert L.mp_plan_create(0, ne, 0, None, g, g, g, g, None, ctypes.byref(out)) == mp.MP_ERR_INVALID
    for dt in (7, -5, 2 ** 31 - 1, -2 ** 31):             # any int32 is refused cleanly
        assert L.mp_plan_create(1, ne, dt, None, g, g, g, g, None, ctypes.byref(out)) == mp.MP_ERR_INVALID
    assert mp.mp_status_string(99) == "MP_ERR_UNKNOWN" and mp.mp_status_string(-1) == "MP_ERR_UNKNOWN"
    assert L.mp_plan_create(1, ne, 0, None, None, g, g, g, None, ctypes.byref(out)) == mp.MP_ERR_INVALID
    assert (L.mp_plan_create(1, ne, 0, None, ctypes.cast(bad, PP), g, g, g, None, ctypes.byref(out))
            == mp.MP_ERR_ALIGN)
    assert "aligned" in mp.mp_last_error()
    zero = (ctypes.c_int64 * 1)(0)
    assert L.mp_plan_create(1, zero, 0, None, g, g, g, g, None, ctypes.byref(out)) == mp.MP_ERR_INVALID
    # more than 2^48 elements in one plan is refused before any allocation
    big_n = 300
    big = (ctypes.c_int64 * big_n)(*([2 ** 40] * big_n))
    gp = ctypes.cast((ctypes.c_void_p * big_n)(*([0x10000] * big_n)), PP)
    assert L.mp_plan_create(big_n, big, 0, None, gp, gp, gp, gp, None, ctypes.byref(out)) == mp.MP_ERR_INVALID
    assert "2^48" in mp.mp_last_error()
    # more chunks than a launch grid holds (2^42 elements in 2048-element chunks) is refused
    # before the chunk table is built, by the plan and by the host-only layout call
    four = (ctypes.c_int64 * 4)(*([2 ** 40] * 4))
    g4 = ctypes.cast((ctypes.c_void_p * 4)(*([0x10000] * 4)), PP)
    assert L.mp_plan_create(4, four, 0, None, g4, g4, g4, g4, None, ctypes.byref(out)) == mp.MP_ERR_INVALID
    assert "2^31" in mp.mp_last_error()
    assert L.mp_chunk_layout(4, four, 256, None, None, None, None, None, 0) == mp.MP_ERR_INVALID
    neg = (ctypes.c_float * 1)(-1.0)
    assert L.mp_plan_create(1, ne, 0, None, g, g, g, g, neg, ctypes.byref(out)) == mp.MP_ERR_INVALID
    for cfg in (mp.scaler_cfg(init_scale=3.0), mp.scaler_cfg(growth=0.5), mp.scaler_cfg(backoff=2.0),
                mp.scaler_cfg(interval=0), mp.scaler_cfg(min_scale=2.0 ** 20),
                mp.scaler_cfg(init_scale=float("inf"))):
        assert L.mp_state_create(ctypes.byref(cfg), ctypes.byref(out)) == mp.MP_ERR_INVALID
    assert L.mp_accumulate(None, None, 1.0, 1, None) == mp.MP_ERR_INVALID
    assert L.mp_unscale_check_norm(None, None, None, 1.0, 0, 1.0, None) == mp.MP_ERR_INVALID
    assert L.mp_scaler_update(None, None) == mp.MP_ERR_INVALID
    assert L.mp_cast_to_16(None, None, -1, 0, None) == mp.MP_ERR_INVALID
    assert L.mp_cast_to_16(ctypes.c_void_p(0x10004), ctypes.c_void_p(0x10000), 4, 0,
                           None) == mp.MP_ERR_ALIGN
    assert L.mp_cast_to_16(None, None, 0, 0, None) == mp.MP_OK      # empty cast: nothing to do
    # a foreign or truncated state blob is refused before the state is touched
    fake_state = ctypes.c_void_p(0x10000)
    blob = ctypes.create_string_buffer(mp.MP_STATE_BLOB_BYTES)
    assert L.mp_state_import(fake_state, blob, mp.MP_STATE_BLOB_BYTES, None) == mp.MP_ERR_INVALID
    assert L.mp_state_import(fake_state, blob, 16, None) == mp.MP_ERR_INVALID
    assert L.mp_state_export(fake_state, blob, 16, None) == mp.MP_ERR_INVALID
    assert L.mp_norm_finish(None, None, None, 1.0, None) == mp.MP_ERR_INVALID
    assert L.mp_fp8set_create(None, None, None, ctypes.byref(out)) == mp.MP_ERR_INVALID
    assert L.mp_adamw_step_fp8(None, None, None, 1.0, 0, None, None, None) == mp.MP_ERR_INVALID
    assert L.mp_fp8set_destroy(None) == mp.MP_OK
    assert L.mp_gradset_update(None, None, None) == mp.MP_ERR_INVALID
    assert L.mp_update_step(None, None, None, 1.0, 0, 1.0, None, None) == mp.MP_ERR_INVALID
    assert (L.mp_norm_partial(fake_state, fake_state, None, 1.0, 0, ctypes.c_void_p(0x10001), None)
            == mp.MP_ERR_INVALID)
    # device-weight entry points: NULL, k and alignment checks come before any launch
    dev = ctypes.c_void_p(0x10000)
    assert L.mp_token_weights_dev(0, dev, dev, None) == mp.MP_ERR_INVALID
    assert L.mp_token_weights_dev(2, None, dev, None) == mp.MP_ERR_INVALID
    assert L.mp_token_weights_dev(2, ctypes.c_void_p(0x10004), dev, None) == mp.MP_ERR_ALIGN
    assert L.mp_token_weights_dev(2, dev, ctypes.c_void_p(0x10002), None) == mp.MP_ERR_ALIGN
    # group entry points: the group's size, NULL arrays and NULL members are refused first
    PP = ctypes.POINTER(ctypes.c_void_p)
    two = ctypes.cast((ctypes.c_void_p * 2)(0x10000, None), PP)
    wts = (ctypes.c_float * 2)(0.5, 0.5)
    for n in (0, 5, -1):
        assert L.mp_accumulate_group(fake_state, two, wts, n, 0, 1, None) == mp.MP_ERR_INVALID
        assert (L.mp_update_step_group(fake_state, fake_state, two, wts, n, 0, 1, 1.0, None, None)
                == mp.MP_ERR_INVALID)
    assert L.mp_accumulate_group(fake_state, None, wts, 2, 0, 1, None) == mp.MP_ERR_INVALID
    assert L.mp_accumulate_group(fake_state, two, None, 2, 0, 1, None) == mp.MP_ERR_INVALID
    assert L.mp_accumulate_group(None, two, wts, 2, 0, 1, None) == mp.MP_ERR_INVALID
    assert (L.mp_update_step_group(None, None, two, wts, 2, 0, 1, 1.0, None, None)
            == mp.MP_ERR_INVALID)
    for n in (0, 5):
        assert (L.mp_unscale_check_norm_group(fake_state, fake_state, two, wts, n, 0, 0, 1.0, None)
                == mp.MP_ERR_INVALID)
        assert (L.mp_adamw_step_group(fake_state, fake_state, two, wts, n, 0, 0, None, None)
                == mp.MP_ERR_INVALID)
    assert L.mp_unscale_check_norm_group(None, None, two, wts, 2, 0, 0, 1.0, None) == mp.MP_ERR_INVALID
    assert L.mp_adamw_step_group(None, None, two, wts, 2, 0, 0, None, None) == mp.MP_ERR_INVALID
    assert L.mp_adamw_step_group(fake_state, fake_state, None, wts, 1, 0, 0, None, None) == mp.MP_ERR_INVALID
    for n in (0, 5):
        assert (L.mp_norm_partial_group(fake_state, fake_state, two, wts, n, 0, 0,
                                        ctypes.c_void_p(0x10000), None) == mp.MP_ERR_INVALID)
    assert (L.mp_norm_partial_group(None, None, two, wts, 1, 0, 0, ctypes.c_void_p(0x10000), None)
            == mp.MP_ERR_INVALID)
    # the first accumulation with counts: NULL arrays, n and k ranges, alignment (the plan is
    # not touched before these)
    fc = L.mp_accumulate_first_counts
    assert fc(fake_state, None, 1, 4, dev, dev, None) == mp.MP_ERR_INVALID
    assert fc(fake_state, two, 1, 4, None, dev, None) == mp.MP_ERR_INVALID
    assert fc(fake_state, two, 1, 4, dev, None, None) == mp.MP_ERR_INVALID
    for n, k in ((0, 4), (5, 8), (2, 1), (1, 65), (1, 0)):
        assert fc(fake_state, two, n, k, dev, dev, None) == mp.MP_ERR_INVALID, (n, k)
    assert fc(fake_state, two, 1, 4, ctypes.c_void_p(0x10004), dev, None) == mp.MP_ERR_ALIGN
    assert fc(fake_state, two, 1, 4, dev, ctypes.c_void_p(0x10002), None) == mp.MP_ERR_ALIGN
    assert fc(None, two, 1, 4, dev, dev, None) == mp.MP_ERR_INVALID


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asking for more exits with a message (no GPU touched)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
