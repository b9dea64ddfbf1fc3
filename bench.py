"""Throughput of the fused mixed-precision update step on one MI355X.

One step = one logical update of the whole hot path over one batch of synthetic
input: micro-batches 1..k-1 accumulated into the fp32 buffers (the token
weights computed from device-resident target counts inside the first of those
passes), the last micro-batch
folded into the unscale/overflow/norm pass and into the AdamW + RNE-cast pass,
then the loss-scaler decision.  Inputs (fp32 masters,
per-micro-batch bf16 gradients) are generated on the device before the timed
region and stay resident in HBM.

Prints ONE JSON line: params/s of the whole step (value), the roofline of the
dominant kernel (the AdamW pass, timed live with HIP events on the stream it
runs on), the fused step (norm + AdamW + scaler, the two passes over the final
gradient) in GB/s, and the oracle timed on the host's cores over a bounded
sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cold] [--graph] [--gpus 1]
"""
import argparse
import ctypes
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "fused mixed-precision step: params/sec and HBM GB/s (% of peak), 1 MI355X"
# the device code the counters measure (the host half of the library does not change it)
KERNEL_SOURCES = [os.path.join(ROOT, "optimizer_step_tensor_amd", "csrc", f)
                  for f in ("internal.h", "kernels.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_llama3-8B.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bytes_per_param(k):
    """Algorithmic HBM bytes per parameter of each pass (16-bit = 2 B, fp32 = 4 B)."""
    return {
        "accumulate_first": 2 + 4,            # read g16, write acc
        "accumulate": 2 + 4 + 4,              # read g16 + acc, write acc
        "norm": (4 if k > 1 else 0) + 2,      # read acc (k > 1) + last g16
        # read acc (k > 1), last g16, w, m, v; write w, m, v, w16
        "adamw": (4 if k > 1 else 0) + 2 + 4 + 4 + 4 + (4 + 4 + 4 + 2),
        "step": (6 + 10 * (k - 2) + 6 + 32) if k >= 2 else (2 + 2 + 4 * 3 + 12 + 2),
    }


def launches_per_step(k, n_chunks, one_call):
    """Kernel launches of one step as bench.py enqueues it: the k - 1 accumulate passes (the
    token weights computed inside the first, or their own launch when k = 1), the norm's first
    stage, its second stage when there are more than 8192 partial sums, its finish, AdamW, then
    the clock and the scaler (their own launches unless one call lets the norm's finish take
    them)."""
    n = (k - 1) if k > 1 else 1
    partials = n_chunks if k > 1 else (n_chunks + 15) // 16   # one stream: 16 chunks per block
    n += 1 + (1 if partials > 8192 else 0) + 1 + 1
    n += 0 if one_call else 2
    return n


def cpu_baseline(w, seconds_hint=20.0):
    """The oracle (as it stands) on a bounded sample: layer-0-sized tensors of the workload,
    split into 16M-element segments so the host threads share the work."""
    import numpy as np
    import inputs
    import oracle
    threads = min(16, os.cpu_count() or 1)
    # sample: the tensors of the first transformer layer (after the embedding)
    sample, total = [], 0
    for t, n in enumerate(w.numels[1:], start=1):
        sample.append((t, n))
        total += n
        if total >= 200_000_000 or len(sample) >= 9:
            break
    seg = 16 * 1024 * 1024
    pieces = []
    for t, n in sample:
        for off in range(0, n, seg):
            pieces.append((t, off, min(seg, n - off)))
    dt = oracle.BF16
    masters = [inputs.gen_host_f32(c, w.master_recipe(t), off) for t, off, c in pieces]
    st = oracle.OracleStep(dt, masters, [np.zeros(x.size, np.uint16) for x in masters],
                           with_acc=w.k > 1, threads=threads)
    grads = [[inputs.gen_host_u16(c, w.grad_recipe(1, i, t), w.dtype, off)
              for t, off, c in pieces] for i in range(w.k)]
    weights = oracle.token_weights(w.token_counts(1))
    t0, c0 = time.perf_counter(), time.process_time()
    for i in range(w.k - 1):
        st.accumulate(grads[i], weights[i], i == 0)
    st.unscale_check_norm(grads[-1], weights[-1], w.k == 1, w.max_norm)
    st.adamw_step(grads[-1], weights[-1], w.k == 1, **w.hp)
    st.scaler_update()
    dt_s = time.perf_counter() - t0
    cpu_s = time.process_time() - c0            # CPU time of all threads of this process
    n_sample = sum(p[2] for p in pieces)
    # the same oracle on one thread, over one 16M-element segment
    j = max(range(len(pieces)), key=lambda i: pieces[i][2])
    one = oracle.OracleStep(dt, [masters[j].copy()], [np.zeros(masters[j].size, np.uint16)],
                            with_acc=w.k > 1, threads=1)
    t1 = time.perf_counter()
    for i in range(w.k - 1):
        one.accumulate([grads[i][j]], weights[i], i == 0)
    one.unscale_check_norm([grads[-1][j]], weights[-1], w.k == 1, w.max_norm)
    one.adamw_step([grads[-1][j]], weights[-1], w.k == 1, **w.hp)
    one.scaler_update()
    dt_1 = time.perf_counter() - t1
    return {"value": n_sample / dt_s, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": "%d params (%d tensors of the first layer, %d segments), k=%d, one full step, "
                      "%.1f s wall, %.1f s of CPU time" % (n_sample, len(sample), len(pieces), w.k,
                                                            dt_s, cpu_s),
            "cpu_seconds": cpu_s,
            "single_thread": {"value": masters[j].size / dt_1, "unit": "params/s",
                              "sample": "one segment (%d params), %.2f s"
                                        % (masters[j].size, dt_1)}}


def kernel_sha():
    """Digest of the library sources: counter results are only reused for identical code."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per AdamW launch from the committed rocprofv3 counter runs, if they were taken
    on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def time_launches(torch, stream, fn, reps):
    """Average ms of `reps` calls of fn, HIP events on the library's stream."""
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_fused_fp8(mp, torch, w, model, sets, state, hp, weights, stream, reps=3):
    """AdamW with the block-16 FP8 cast of every tensor whose size allows it, fused, and the
    plain AdamW pass, each timed with HIP events around its own launch."""
    k = w.k
    offs, total = [], 0
    for n in w.numels:
        offs.append(total)
        total += (n + 127) // 128 * 128               # every code array on a 128-byte line
    codes = torch.empty(total, dtype=torch.uint8, device="cuda")
    scales = torch.empty(total // 16, dtype=torch.float32, device="cuda")
    cv = [codes[o:o + n] if n % 16 == 0 else None for o, n in zip(offs, w.numels)]
    sv = [scales[o // 16:o // 16 + n // 16] if n % 16 == 0 else None
          for o, n in zip(offs, w.numels)]
    n_cast = sum(n for n in w.numels if n % 16 == 0)
    fs = mp.mp_fp8set_create(model.plan, cv, sv)
    lif = k == 1
    times = {"fused": [], "plain": []}
    try:
        for _ in range(reps + 1):
            for kind in ("fused", "plain"):
                mp.mp_unscale_check_norm(model.plan, state, sets[-1], weights[-1], lif, w.max_norm,
                                         stream)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                if kind == "fused":
                    mp.mp_adamw_step_fp8(model.plan, state, sets[-1], weights[-1], lif, hp, fs,
                                         stream)
                else:
                    mp.mp_adamw_step(model.plan, state, sets[-1], weights[-1], lif, hp, stream)
                e1.record(stream)
                mp.mp_scaler_update(state, stream)
                times[kind].append((e0, e1))
        torch.cuda.synchronize()
    finally:
        mp.mp_fp8set_destroy(fs)
    ms = {kind: sum(a.elapsed_time(b) for a, b in v[1:]) / reps for kind, v in times.items()}
    adam_bpp = bytes_per_param(k)["adamw"]
    fused_bytes = adam_bpp * w.total + 1.25 * n_cast
    return {"elements_cast": n_cast, "ms": ms["fused"], "plain_adamw_ms": ms["plain"],
            "extra_ms": ms["fused"] - ms["plain"], "bytes": fused_bytes,
            "GBps": fused_bytes / ms["fused"] / 1e6,
            "frac": fused_bytes / ms["fused"] / 1e6 / HBM_PEAK_GBPS}


def time_save_restore(mp, torch, state, stream, reps=20):
    """Export of the device state into pinned host memory (enqueue + wait) and import of the
    blob back (validated on the host, copied, waited for), host wall time per call."""
    blob = torch.empty(mp.MP_STATE_BLOB_BYTES, dtype=torch.uint8, pin_memory=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        mp.mp_state_export(state, blob.data_ptr(), mp.MP_STATE_BLOB_BYTES, stream)
        stream.synchronize()
    t1 = time.perf_counter()
    for _ in range(reps):
        mp.mp_state_import(state, blob.data_ptr(), mp.MP_STATE_BLOB_BYTES, stream)
    t2 = time.perf_counter()
    return {"blob_bytes": mp.MP_STATE_BLOB_BYTES, "export_us": (t1 - t0) / reps * 1e6,
            "import_us": (t2 - t1) / reps * 1e6}


EXTRAS = ("device_copy", "fp8_block_cast", "adamw_fp8_fused", "state_save_restore",
          "zero8_rank_share", "resident_groups", "ceiling")


def flat_extent(model, arrays):
    """(base address, element count) of each flat buffer behind a flat-layout model's views."""
    from optimizer_step_tensor_amd import _align_elems
    n = sum(_align_elems(x) for x in model.numels)
    return [(a[0].data_ptr(), n) for a in arrays], n


def time_ceiling(torch, w, model, g16_last, stream, kernel_ms, reps=3):
    """Bandwidth probes (optimizer_step_tensor_amd/csrc/ceiling.hip) over the model's own flat
    buffers, in the library's launch shape: the AdamW pass's exact traffic (5 streams read,
    4 written, trivial arithmetic, state left as it was) at several caps on resident blocks
    per CU, the norm's read traffic, the first and the later accumulations' traffic into the
    (dead) accumulator, and a copy and a fill of it.  Each pass of the step is rated against
    the fastest probe of its own pattern."""
    from optimizer_step_tensor_amd import build as lib_build
    if model.layout != "flat" or model.acc is None:
        return {"skipped": "needs the flat layout and an accumulator"}
    C = ctypes.CDLL(lib_build.CEILING_LIB)
    i64, i32, P_, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
    C.mpc_adamw_pattern.argtypes = [P_, P_, P_, P_, P_, P_, i64, i32, i32, i32, P_]
    C.mpc_read_pattern.argtypes = [P_, P_, i64, P_, i32, i32, P_]
    C.mpc_copy_pattern.argtypes = [P_, P_, i64, i32, i32, P_]
    C.mpc_fill_pattern.argtypes = [P_, i64, f32, i32, i32, P_]
    C.mpc_accumulate_pattern.argtypes = [P_, P_, i64, i32, i32, i32, P_]
    for f in (C.mpc_adamw_pattern, C.mpc_read_pattern, C.mpc_copy_pattern, C.mpc_fill_pattern,
              C.mpc_accumulate_pattern):
        f.restype = i32
    (acc, master, m, v, w16, g), n = flat_extent(
        model, [model.acc, model.master, model.m, model.v, model.w16, g16_last])
    acc, master, m, v, w16, g = [x[0] for x in (acc, master, m, v, w16, g)]
    sink = torch.empty((n + 2047) // 2048, dtype=torch.float32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    fp16 = int(model.dtype != 0)

    def timed(fn):
        assert fn() == 0
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            assert fn() == 0
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {"elements": n, "reps": reps, "shape": "one 256-lane block per 2048 elements, "
                                                  "XCD runs of `span` chunks, nontemporal"}
    adam_bytes, read_bytes = 32 * n, 6 * n
    pat = {}
    for cap in (0, 3, 4, 5):
        for span in (64, 128):
            ms = timed(lambda: C.mpc_adamw_pattern(acc, g, master, m, v, w16, n, fp16, cap, span,
                                                   sp))
            pat["cap%d_span%d" % (cap, span)] = {"ms": ms, "GBps": adam_bytes / ms / 1e6}
    best = max(pat.values(), key=lambda r: r["GBps"])
    out["adamw_pattern"] = {"bytes_per_element": 32, "runs": pat, "best_GBps": best["GBps"],
                            "best_frac": best["GBps"] / HBM_PEAK_GBPS}
    rd = {}
    for cap in (0,):
        for span in (64, 128):
            ms = timed(lambda: C.mpc_read_pattern(acc, g, n, sink.data_ptr(), cap, span, sp))
            rd["cap%d_span%d" % (cap, span)] = {"ms": ms, "GBps": read_bytes / ms / 1e6}
    best_rd = max(rd.values(), key=lambda r: r["GBps"])
    out["norm_pattern"] = {"bytes_per_element": 6, "runs": rd, "best_GBps": best_rd["GBps"],
                           "best_frac": best_rd["GBps"] / HBM_PEAK_GBPS}
    # the accumulator is dead between steps (the next first accumulation overwrites it)
    for name, fn, bpe in (
            ("first_accumulate_pattern",
             lambda cap, span: C.mpc_accumulate_pattern(acc, g, n, 0, cap, span, sp), 6),
            ("accumulate_pattern",
             lambda cap, span: C.mpc_accumulate_pattern(acc, g, n, 1, cap, span, sp), 10),
            ("copy_in_place", lambda cap, span: C.mpc_copy_pattern(acc, acc, n, cap, span, sp), 8),
            ("fill", lambda cap, span: C.mpc_fill_pattern(acc, n, 0.0, cap, span, sp), 4)):
        runs = {}
        for cap in (0, 4):
            for span in (64, 128):
                ms = timed(lambda: fn(cap, span))
                runs["cap%d_span%d" % (cap, span)] = {"ms": ms, "GBps": bpe * n / ms / 1e6}
        b = max(runs.values(), key=lambda r: r["GBps"])
        out[name] = {"bytes_per_element": bpe, "runs": runs, "best_GBps": b["GBps"],
                     "best_frac": b["GBps"] / HBM_PEAK_GBPS}
    P = w.total
    step_adam = 32 * P / kernel_ms["adamw"] / 1e6
    step_norm = 6 * P / kernel_ms["norm"] / 1e6
    out["adamw_vs_pattern"] = step_adam / best["GBps"]
    out["norm_vs_pattern"] = step_norm / best_rd["GBps"]
    out["first_accumulate_vs_pattern"] = (6 * P / kernel_ms["first_accumulate"] / 1e6 /
                                          out["first_accumulate_pattern"]["best_GBps"])
    if kernel_ms.get("accumulate"):
        out["accumulate_vs_pattern"] = (10 * P / kernel_ms["accumulate"] / 1e6 /
                                        out["accumulate_pattern"]["best_GBps"])
    # the fused step at the speed of its two patterns
    t_ceil = adam_bytes / best["GBps"] / 1e6 + read_bytes / best_rd["GBps"] / 1e6
    out["fused_step_pattern_frac"] = (adam_bytes + read_bytes) / t_ceil / 1e6 / HBM_PEAK_GBPS
    return out


def run_extras(mp, torch, w, model, g16, sets, state, hp, weights, stream, only=None,
               kernel_ms=None):
    """The rows after the hot path, on the same resident buffers (`only`: a subset of EXTRAS):
    - the runtime's own device-to-device copy of 4 GiB, context for the roofline;
    - the fine-grained FP8 cast (block 16) of every fp32 master;
    - the same cast fused into the AdamW pass (mp_adamw_step_fp8), against the plain AdamW pass
      timed the same way in alternation;
    - saving and restoring the device state (scaler and optimizer clock);
    - one rank's share of a ZeRO-8 step: a plan over 1/8 of every tensor (slice boundaries on
      multiples of 64 elements), its accumulate passes, partial norm + finish, AdamW, scaler;
    - the step with all k micro-batch gradients resident, folded in groups of up to four
      (time_groups).  Same results, bit for bit, as the timed step;
    - bandwidth probes of the AdamW and norm access patterns at the model's size (time_ceiling),
      last, since the fill probe overwrites the dead accumulator."""
    def want(name):
        return only is None or name in only

    out = {}
    if want("device_copy"):
        a = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        ms = time_launches(torch, stream, lambda: b.copy_(a), 5)
        out["device_copy"] = {"bytes_read": 4 << 30, "bytes_written": 4 << 30, "ms": ms,
                              "GBps": 2 * (4 << 30) / ms / 1e6,
                              "frac": 2 * (4 << 30) / ms / 1e6 / HBM_PEAK_GBPS}
        del a, b
    if want("fp8_block_cast"):
        out["fp8_block_cast"] = time_fp8_cast(mp, torch, w, model, stream)
    if want("adamw_fp8_fused"):
        out["adamw_fp8_fused"] = time_fused_fp8(mp, torch, w, model, sets, state, hp, weights,
                                                stream)
    if want("state_save_restore"):
        out["state_save_restore"] = time_save_restore(mp, torch, state, stream)
    if want("zero8_rank_share"):
        out["zero8_rank_share"] = time_rank_share(mp, torch, w, model, g16, hp, weights, stream)
    if want("resident_groups") and w.k >= 2:
        out["resident_groups"] = time_groups(mp, torch, w, model, sets, state, hp, weights,
                                             stream)
    if want("ceiling") and kernel_ms is not None and w.k >= 2:
        out["ceiling"] = time_ceiling(torch, w, model, g16[-1], stream, kernel_ms)
    return out


def time_fp8_cast(mp, torch, w, model, stream):
    big = max(w.numels)
    codes = torch.empty(big, dtype=torch.uint8, device="cuda")
    scales = torch.empty(big // 16 + 1, dtype=torch.float32, device="cuda")
    cast = [(x, n - n % 16) for x, n in zip(model.master, w.numels) if n >= 16]

    def fp8_all():
        for x, n in cast:
            mp.mp_cast_fp8_blocks(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), n, 16, stream)

    ms = time_launches(torch, stream, fp8_all, 3)
    n_cast = sum(n for _, n in cast)
    gbps = n_cast * (4 + 1 + 4 / 16) / ms / 1e6
    return {"block": 16, "elements": n_cast, "ms": ms, "bytes_per_element": 5.25, "GBps": gbps,
            "frac": gbps / HBM_PEAK_GBPS}


def time_rank_share(mp, torch, w, model, g16, hp, weights, stream):
    k = w.k
    ranks, r = 8, 0
    numel, ptrs = [], {"acc": [], "master": [], "m": [], "v": [], "w16": []}
    gp = [[] for _ in range(k)]
    for t, n in enumerate(w.numels):
        per = mp._align_elems((n + ranks - 1) // ranks)   # ceil(n / ranks), rounded up to 64
        lo, hi = min(n, r * per), min(n, (r + 1) * per)
        if hi <= lo:
            continue
        numel.append(hi - lo)
        for name, esz in (("acc", 4), ("master", 4), ("m", 4), ("v", 4), ("w16", 2)):
            ptrs[name].append(getattr(model, name)[t].data_ptr() + esz * lo)
        for i in range(k):
            gp[i].append(g16[i][t].data_ptr() + 2 * lo)
    plan = mp.mp_plan_create(numel, model.dtype, ptrs["acc"], ptrs["master"], ptrs["m"],
                             ptrs["v"], ptrs["w16"])
    sets = [mp.mp_gradset_create(plan, g) for g in gp]
    st = mp.mp_state_create(mp.scaler_cfg(init_scale=1.0, enabled=False))
    part = torch.zeros(1, dtype=torch.float64, device="cuda")

    def shard_step():
        for i in range(k - 1):
            mp.mp_accumulate(plan, sets[i], weights[i], i == 0, stream)
        mp.mp_norm_partial(plan, st, sets[-1], weights[-1], k == 1, part.data_ptr(), stream)
        # (the all-reduce of the one partial sum would run here)
        mp.mp_norm_finish(plan, st, part.data_ptr(), w.max_norm, stream)
        mp.mp_adamw_step(plan, st, sets[-1], weights[-1], k == 1, hp, stream)
        mp.mp_scaler_update(st, stream)

    ms = time_launches(torch, stream, shard_step, 3)
    p_share = sum(numel)
    for g in sets:
        mp.mp_gradset_destroy(g)
    mp.mp_state_destroy(st)
    mp.mp_plan_destroy(plan)
    return {"params": p_share, "ms_per_step": ms, "params_per_s": p_share / (ms * 1e-3),
            "GBps": bytes_per_param(k)["step"] * p_share / ms / 1e6}


def group_bytes_per_param(acc_groups, fold):
    """Algorithmic bytes per parameter of one step folded in groups: an accumulate pass of n
    micro-batches reads 2n (+4 for the accumulator unless it is the first) and writes 4; the
    norm reads 2n (+4) and AdamW 2n (+4) + 12 and writes 14, the +4 when the step has an
    accumulator."""
    b = sum(2 * len(g) + (4 if i == 0 else 8) for i, g in enumerate(acc_groups))
    acc = 4 if acc_groups else 0
    return b + (acc + 2 * len(fold)) + (acc + 2 * len(fold) + 12 + 14)


def time_groups(mp, torch, w, model, sets, state, hp, weights, stream, reps=3):
    """k <= 4: all micro-batches folded into the norm and AdamW passes, and (k >= 3) the first
    two accumulated in one pass with the rest folded.  k > 4: the first k - 4 accumulated in
    groups of up to four, the last four folded.  Each schedule is timed eagerly (host weights)
    and as a captured step replayed (token weights computed on the device from device counts,
    every pass reading its weights there)."""
    k = w.k
    counts_dev = torch.tensor(w.token_counts(1), dtype=torch.int64, device="cuda")
    wdev = torch.empty(k, dtype=torch.float32, device="cuda")
    schedules = {}
    if k <= 4:
        schedules["all_folded"] = ([], list(range(k)))
        if k >= 3:
            schedules["two_accumulated"] = ([[0, 1]], list(range(2, k)))
    else:
        head = list(range(k - 4))
        schedules["groups_of_four"] = ([head[i:i + 4] for i in range(0, len(head), 4)],
                                       list(range(k - 4, k)))
    out = {}
    for name, (acc_groups, fold) in schedules.items():
        def step():
            for i, g in enumerate(acc_groups):
                mp.mp_accumulate_group(model.plan, [sets[j] for j in g], [weights[j] for j in g],
                                       i == 0, stream)
            mp.mp_update_step_group(model.plan, state, [sets[j] for j in fold],
                                    [weights[j] for j in fold], not acc_groups, w.max_norm, hp,
                                    stream)
        ms = time_launches(torch, stream, step, reps)
        bpp = group_bytes_per_param(acc_groups, fold)

        def device_step(s):
            mp.mp_token_weights_dev(k, counts_dev, wdev, s)
            for i, g in enumerate(acc_groups):
                mp.mp_accumulate_group(model.plan, [sets[j] for j in g],
                                       wdev.data_ptr() + 4 * g[0], i == 0, s)
            mp.mp_update_step_group(model.plan, state, [sets[j] for j in fold],
                                    wdev.data_ptr() + 4 * fold[0], not acc_groups, w.max_norm, hp,
                                    s)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            device_step(torch.cuda.current_stream())
        gms = time_launches(torch, stream, graph.replay, 10 * reps)
        del graph
        out[name] = {"schedule": {"accumulated": acc_groups, "folded": fold},
                     "bytes_per_param": bpp, "ms_per_step": ms,
                     "params_per_s": w.total / (ms * 1e-3),
                     "GBps": bpp * w.total / ms / 1e6,
                     "frac": bpp * w.total / ms / 1e6 / HBM_PEAK_GBPS,
                     "graph_ms_per_step": gms,
                     "graph_frac": bpp * w.total / gms / 1e6 / HBM_PEAK_GBPS}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3-8B")
    ap.add_argument("--layout", default="flat", choices=("tensor", "flat"),
                    help="one allocation per tensor, or one flat buffer per kind of array")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and replay it (launch-bound workloads)")
    ap.add_argument("--trace-steps", type=int, default=0,
                    help="time this many single steps after warm-up and print each")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements after the hot path (extras)")
    ap.add_argument("--extras", default=None,
                    help="comma-separated subset of the extras to run: " + ", ".join(EXTRAS))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 4 GiB device copy (for counter calibration)")
    ap.add_argument("--cold", action="store_true",
                    help="overwrite a 1 GiB scratch buffer before every timed step (evicts the "
                         "state of small workloads from the last-level cache) and time each step "
                         "with its own events")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    only = None
    if args.extras:
        only = set(args.extras.split(","))
        unknown = only - set(EXTRAS)
        if unknown:
            print("unknown extras: %s (known: %s)" % (", ".join(sorted(unknown)), ", ".join(EXTRAS)),
                  file=sys.stderr)
            sys.exit(2)

    import torch
    import inputs
    import optimizer_step_tensor_amd as mp
    from inputs import configs

    w = configs.make(args.workload)
    P, k = w.total, w.k
    log("workload %s: %d tensors, %d params, k=%d" % (w.name, len(w.tensors), P, k))
    torch.cuda.set_device(0)
    dt16 = mp.MP_BF16 if w.dtype == inputs.BF16 else mp.MP_FP16
    t16 = torch.bfloat16 if w.dtype == inputs.BF16 else torch.float16
    model = mp.ModelState(w.numels, dt16, with_acc=k > 1, layout=args.layout)
    for t, x in enumerate(model.master):
        inputs.fill_dev_f32(x, w.master_recipe(t))
    for x, y in zip(model.master, model.w16):
        mp.mp_cast_to_16(x.data_ptr(), y.data_ptr(), x.numel(), dt16)
    cfg = (mp.scaler_cfg(**w.scaler) if w.scaler is not None
           else mp.scaler_cfg(init_scale=1.0, enabled=False))
    state = mp.mp_state_create(cfg)
    S0 = cfg.init_scale
    g16 = []
    for i in range(k):
        g16.append(model.grad_buffers())
        for t, x in enumerate(g16[-1]):
            inputs.fill_dev_u16(x, w.grad_recipe(1, i, t, S0), w.dtype)
    sets = [model.gradset(g) for g in g16]
    hp = mp.adamw_hparams(**w.hp)
    counts = w.token_counts(1)
    weights = mp.mp_token_weights(counts)        # host weights, for the extras
    plan = model.plan
    stream = torch.cuda.current_stream()
    # the step's token weights are computed on the device from device-resident counts, and
    # every pass reads its weight there: the whole step is stream-ordered device work
    counts_dev = torch.tensor(counts, dtype=torch.int64, device="cuda")
    weights_dev = torch.empty(k, dtype=torch.float32, device="cuda")
    # the timed loop calls the C ABI directly with arguments marshalled once here, so no
    # per-call ctypes array building lands in the step time of the small workloads
    L = mp.lib()
    PP = ctypes.POINTER(ctypes.c_void_p)
    one = [ctypes.cast((ctypes.c_void_p * 1)(x.value), PP) for x in sets]   # groups of one
    wptr = [ctypes.c_void_p(weights_dev.data_ptr() + 4 * i) for i in range(k)]
    cptr, wdev = ctypes.c_void_p(counts_dev.data_ptr()), ctypes.c_void_p(weights_dev.data_ptr())
    info = mp.mp_plan_info(plan)
    log("plan:", info, "| resident %.1f GB" % (torch.cuda.memory_allocated() / 1e9))

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read, %d bytes written" % (4 * n, 4 * n))
        del a, b

    ev = {name: [] for name in ("first_accumulate", "accumulate", "norm", "adamw", "fused")}
    # every timing event is created, and recorded once so that its HIP event exists, before
    # any timed region; the timed steps then only record them
    pool = [torch.cuda.Event(enable_timing=True)
            for _ in range(args.steps * (2 * k + 6) + 2)]
    for e in pool:
        e.record(stream)
    torch.cuda.synchronize()
    pool.reverse()
    take = pool.pop

    def one_step_on(stream, record, one_call=False):
        """One step: the accumulations (the first computing the token weights from the device
        counts, or their own launch when k = 1), then the norm, AdamW and the scaler.  Eager steps call those three separately, with events around
        each; a captured step (one_call) enqueues them with mp_update_step_group, whose norm
        finish also takes the clock and the scaler's decision (fewest launches)."""
        def timed(name, fn):
            if record:
                e0 = take()
                e1 = take()
                e0.record(stream)
                fn()
                e1.record(stream)
                ev[name].append((e0, e1))
            else:
                fn()
        lif = int(k == 1)
        sp = ctypes.c_void_p(stream.cuda_stream)
        chk = mp._check
        if k == 1:
            chk(L.mp_token_weights_dev(k, cptr, wdev, sp))
        for i in range(k - 1):
            if i == 0:                        # the token weights are computed in this pass
                timed("first_accumulate",
                      lambda: chk(L.mp_accumulate_first_counts(plan, one[0], 1, k, cptr, wdev, sp)))
            else:
                timed("accumulate",
                      lambda i=i: chk(L.mp_accumulate_group(plan, one[i], wptr[i], 1, 1, 0, sp)))
        if one_call:
            chk(L.mp_update_step_group(plan, state, one[-1], wptr[-1], 1, 1, lif, w.max_norm,
                                       ctypes.byref(hp), sp))
            return
        if record:                            # the fused step: norm + AdamW + scaler
            f0 = take()
            f0.record(stream)
        timed("norm", lambda: chk(L.mp_unscale_check_norm_group(plan, state, one[-1], wptr[-1], 1,
                                                                 1, lif, w.max_norm, sp)))
        timed("adamw", lambda: chk(L.mp_adamw_step_group(plan, state, one[-1], wptr[-1], 1, 1,
                                                         lif, ctypes.byref(hp), sp)))
        chk(L.mp_scaler_update(state, sp))
        if record:
            f1 = take()
            f1.record(stream)
            ev["fused"].append((f0, f1))

    graph = None
    if args.graph:
        # the step is stream-ordered with no host sync: capture it once and replay it
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            one_step_on(torch.cuda.current_stream(), False, one_call=True)

    def one_step(record):
        if graph is not None:
            graph.replay()
        else:
            one_step_on(stream, record)

    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()
    if args.trace_steps:
        for i in range(args.trace_steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            one_step(False)
            b.record(stream)
            b.synchronize()
            log("trace step %d: %.3f ms" % (i, a.elapsed_time(b)))
    # eager steps carry HIP events around every launch, on the stream the library launches
    # on, inside the timed region; a replayed graph cannot, so after a graph run the same
    # number of eager steps is timed with events outside it
    record = graph is None
    gc.collect()
    gc.disable()                              # no collector pauses inside the timed region
    if args.cold:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        step_ms = []
        for _ in range(args.steps):
            flush.fill_(1.0)
            a = take()
            b = take()
            a.record(stream)
            one_step(record)
            b.record(stream)
            b.synchronize()
            step_ms.append(a.elapsed_time(b))
        ms_per_step = sum(step_ms) / len(step_ms)
        del flush
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        bounds = [take() for _ in range(args.steps + 1)]
        bounds[0].record(stream)
        for i in range(args.steps):
            one_step(record)
            bounds[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = bounds[0].elapsed_time(bounds[-1])
        ms_per_step = max(wall * 1e3, gpu_ms) / args.steps
        step_ms = [a.elapsed_time(b) for a, b in zip(bounds, bounds[1:])]
    stats = mp.read_stats(state)
    log("stats after timing:", stats)

    bpp = bytes_per_param(k)
    if not record:
        for _ in range(args.steps):
            one_step_on(stream, True)
    torch.cuda.synchronize()
    gc.enable()
    kernel_ms = {n: (sum(a.elapsed_time(b) for a, b in v) / len(v) if v else None)
                 for n, v in ev.items()}
    adam_bytes = bpp["adamw"] * P
    achieved = adam_bytes / (kernel_ms["adamw"] * 1e-3) / 1e9
    step_bytes = bpp["step"] * P
    fused_bpp = bpp["norm"] + bpp["adamw"]
    fused_gbps = fused_bpp * P / kernel_ms["fused"] / 1e6
    log("per-launch ms:", {n: round(x, 4) for n, x in kernel_ms.items() if x})
    log("fused step (norm + AdamW + scaler): %.3f ms, %.1f GB/s (%.1f%% of %.0f)"
        % (kernel_ms["fused"], fused_gbps, fused_gbps / HBM_PEAK_GBPS * 100, HBM_PEAK_GBPS))
    log("step: %.3f ms, %.1f GB/s algorithmic (%.1f%% of %.0f)"
        % (ms_per_step, step_bytes / ms_per_step / 1e6, step_bytes / ms_per_step / 1e6 /
           HBM_PEAK_GBPS * 100, HBM_PEAK_GBPS))

    extras = None if args.no_extras else run_extras(mp, torch, w, model, g16, sets, state, hp,
                                                    weights, stream, only, kernel_ms)
    traffic = measured_traffic(w.name)
    out = {
        "metric": METRIC,
        "value": P / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded counter-based generator, inputs resident in HBM)",
        "config": {"workload": w.name, "params": P, "tensors": len(w.tensors), "k": k,
                   "layout": args.layout, "graph": bool(args.graph),
                   "cache": "cold (1 GiB overwritten before each step)" if args.cold else "warm",
                   "kernel_events": "inside the timed region" if record else
                                    "eager steps after the timed graph replays",
                   "dtype16": "bf16" if w.dtype == inputs.BF16 else "fp16",
                   "schedule": "k-1 accumulate passes, the first computing the token weights "
                               "from device counts; the "
                               "last micro-batch folded into the norm and AdamW passes" +
                               ("; one call for norm + AdamW + scaler, whose norm finish takes "
                                "the clock and the scaler" if args.graph else ""),
                   "launches_per_step": launches_per_step(k, info["n_chunks"], args.graph),
                   "step_bytes_per_param": bpp["step"],
                   "step_GBps": step_bytes / ms_per_step / 1e6,
                   "step_hbm_frac": step_bytes / ms_per_step / 1e6 / HBM_PEAK_GBPS,
                   "kernel_ms": kernel_ms,
                   "step_ms_median": statistics.median(step_ms),
                   "step_ms_min": min(step_ms), "step_ms_max": max(step_ms),
                   "chunk_elems": info["chunk_elems"], "n_chunks": info["n_chunks"]},
        "roofline": {"bound": "hbm", "kernel": "k_adamw (AdamW + RNE cast, last micro-batch "
                                                "folded in)",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "bytes_per_param": bpp["adamw"],
                     "traffic": traffic},
        "fused_step": {"passes": "unscale/overflow/norm + AdamW/RNE cast + scaler",
                       "bytes_per_param": fused_bpp, "ms": kernel_ms["fused"],
                       "GBps": fused_gbps, "hbm_frac": fused_gbps / HBM_PEAK_GBPS},
        "cpu_baseline": None,
        "extras": extras,
    }
    for s in sets:
        mp.mp_gradset_destroy(s)
    mp.mp_state_destroy(state)
    model.close()
    del g16, model
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on the host cores) ...")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
