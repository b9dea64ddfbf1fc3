"""Drivers that run one workload through the HIP library and through the oracle.

Both sides read the same seeded inputs (``inputs``): the device side fills its
buffers with the generator's HIP twin, the oracle side with its host twin.
Nothing flows from the HIP path into the oracle.  The update schedule is the
same on both sides: micro-batches 1..k-1 accumulated, the last one folded into
the norm and update passes (or, with ``fold_last = False`` on both, all k
accumulated and the norm and update reading the accumulator alone).
"""
import numpy as np

import inputs
import oracle


def oracle_dtype(w):
    return oracle.BF16 if w.dtype == inputs.BF16 else oracle.FP16


INF16 = {inputs.BF16: 0x7F80, inputs.FP16: 0x7C00}


class OracleRun:
    """The workload on host arrays, stepped by the oracle."""

    def __init__(self, w, threads=8):
        self.w = w
        dt = oracle_dtype(w)
        masters = [inputs.gen_host_f32(n, w.master_recipe(t)) for t, n in enumerate(w.numels)]
        w16 = [oracle.rd16(x, dt) for x in masters]
        sc = (oracle.make_scaler(**w.scaler) if w.scaler is not None
              else oracle.make_scaler(init_scale=1.0, enabled=False))
        self.st = oracle.OracleStep(dt, masters, w16, scaler=sc, with_acc=w.k > 1,
                                    wd_mult=getattr(w, "wd_mult", None), threads=threads)
        self.step_no = 0
        self.fold_last = True              # False: accumulate every micro-batch, then norm/AdamW

    def grads(self, step, micro):
        S = self.st.scaler.scale
        g = [inputs.gen_host_u16(n, self.w.grad_recipe(step, micro, t, S), self.w.dtype)
             for t, n in enumerate(self.w.numels)]
        if micro == self.w.k - 1:
            inj = self.w.injection(step)
            if inj is not None:
                g[inj[0]][inj[1]] = INF16[self.w.dtype]
        return g

    def step(self):
        """One logical update; returns the accumulator snapshot before the fold (or None)."""
        self.step_no += 1
        w, st, s = self.w, self.st, self.step_no
        self.prev_master = [x.copy() for x in st.masters]
        self.prev_m = [x.copy() for x in st.m]
        weights = oracle.token_weights(w.token_counts(s))
        if not self.fold_last:
            for i in range(w.k):
                st.accumulate(self.grads(s, i), weights[i], i == 0)
            acc_snapshot = [a.copy() for a in st.acc]
            st.unscale_check_norm(None, 1.0, False, w.max_norm)
            st.adamw_step(None, 1.0, False, **w.hp)
            st.scaler_update()
            return acc_snapshot
        for i in range(w.k - 1):
            st.accumulate(self.grads(s, i), weights[i], i == 0)
        acc_snapshot = [a.copy() for a in st.acc] if st.acc is not None else None
        last = self.grads(s, w.k - 1)
        lif = w.k == 1
        st.unscale_check_norm(last, weights[-1], lif, w.max_norm)
        st.adamw_step(last, weights[-1], lif, **w.hp)
        st.scaler_update()
        return acc_snapshot


class DeviceRun:
    """The workload in device buffers, stepped by libmpstep."""

    def __init__(self, w, sep_grads=True, layout="tensor"):
        import torch
        import optimizer_step_tensor_amd as mp
        self.torch, self.mp, self.w = torch, mp, w
        dt = mp.MP_BF16 if w.dtype == inputs.BF16 else mp.MP_FP16
        self.model = mp.ModelState(w.numels, dt, with_acc=w.k > 1, layout=layout,
                                   wd_mult=getattr(w, "wd_mult", None))
        for t, x in enumerate(self.model.master):
            inputs.fill_dev_f32(x, w.master_recipe(t))
        for x, y in zip(self.model.master, self.model.w16):
            mp.mp_cast_to_16(x.data_ptr(), y.data_ptr(), x.numel(), dt)
        n_sets = w.k if sep_grads else 1
        self.g16 = [self.model.grad_buffers() for _ in range(n_sets)]
        self.gsets = [self.model.gradset(g) for g in self.g16]
        cfg = (mp.scaler_cfg(**w.scaler) if w.scaler is not None
               else mp.scaler_cfg(init_scale=1.0, enabled=False))
        self.state = mp.mp_state_create(cfg)
        self.hp = mp.adamw_hparams(**w.hp)
        self.step_no = 0
        self.fp8set = None                 # set: steps use the fused AdamW + FP8 entry point
        self.one_call = False              # True: steps use mp_update_step
        self.noalloc = False               # with one_call: mp_update_step_noalloc instead
        self.fold_last = True              # False: accumulate every micro-batch, then norm/AdamW
        self.device_weights = False        # True: weights from device counts, steps use the
        self.dev_counts = None             # group entry points (kept alive until the next step)
        self.dev_weights = None
        self.first_counts = False          # with device_weights: the weights computed inside the
                                           # first accumulation (mp_accumulate_first_counts)
        self.separate = False              # with device_weights: norm, AdamW and scaler as three
                                           # group calls instead of mp_update_step_group
        # (accumulate groups, folded group) of micro-batch indices: steps use
        # mp_accumulate_group per group, then mp_update_step_group on the folded one
        self.schedule = None

    def stats(self):
        return self.mp.read_stats(self.state)

    def fill_grads(self, step, scale):
        """Generate every micro-batch's gradients of `step` (with the given loss scale)."""
        w = self.w
        for i in range(w.k):
            gl = self.g16[i % len(self.g16)]
            for t, x in enumerate(gl):
                inputs.fill_dev_u16(x, w.grad_recipe(step, i, t, scale), w.dtype)
            if i == w.k - 1:
                inj = w.injection(step)
                if inj is not None:
                    gl[inj[0]].view(self.torch.int16)[inj[1]] = INF16[w.dtype]

    def step(self, scale, snapshot=False):
        """One logical update with inputs generated at loss scale `scale`."""
        self.step_no += 1
        mp, w, s = self.mp, self.w, self.step_no
        assert len(self.g16) == w.k, "per-micro-batch buffers needed to run a step"
        self.fill_grads(s, scale)
        if self.schedule is not None:
            return self._step_groups(s)
        if self.device_weights:
            return self._step_device_weights(s, snapshot)
        weights = mp.mp_token_weights(w.token_counts(s))
        if not self.fold_last:
            for i in range(w.k):
                mp.mp_accumulate(self.model.plan, self.gsets[i], weights[i], i == 0)
            acc_snapshot = [a.cpu().numpy() for a in self.model.acc] if snapshot else None
            mp.mp_unscale_check_norm(self.model.plan, self.state, None, 1.0, 0, w.max_norm)
            mp.mp_adamw_step(self.model.plan, self.state, None, 1.0, 0, self.hp)
            mp.mp_scaler_update(self.state)
            return acc_snapshot
        for i in range(w.k - 1):
            mp.mp_accumulate(self.model.plan, self.gsets[i], weights[i], i == 0)
        acc_snapshot = ([a.cpu().numpy() for a in self.model.acc]
                        if snapshot and self.model.acc is not None else None)
        last, lif = self.gsets[w.k - 1], w.k == 1
        if self.one_call:
            call = mp.mp_update_step_noalloc if self.noalloc else mp.mp_update_step
            call(self.model.plan, self.state, last, weights[-1], lif, w.max_norm, self.hp)
            return acc_snapshot
        mp.mp_unscale_check_norm(self.model.plan, self.state, last, weights[-1], lif, w.max_norm)
        if self.fp8set is None:
            mp.mp_adamw_step(self.model.plan, self.state, last, weights[-1], lif, self.hp)
        else:
            mp.mp_adamw_step_fp8(self.model.plan, self.state, last, weights[-1], lif, self.hp,
                                 self.fp8set)
        mp.mp_scaler_update(self.state)
        return acc_snapshot

    def _step_groups(self, s):
        """The step with resident micro-batches folded in groups; with device_weights the
        group calls read the weights from mp_token_weights_dev's output."""
        torch, mp, w = self.torch, self.mp, self.w
        acc_groups, fold = self.schedule
        order = [i for g in acc_groups for i in g] + list(fold)
        assert order == list(range(w.k)), self.schedule
        counts = w.token_counts(s)
        if self.device_weights:
            self.dev_counts = torch.tensor(counts, dtype=torch.int64, device="cuda")
            self.dev_weights = torch.empty(w.k, dtype=torch.float32, device="cuda")
            mp.mp_token_weights_dev(w.k, self.dev_counts, self.dev_weights)

            def wts(grp):
                return self.dev_weights.data_ptr() + 4 * grp[0]
        else:
            host = mp.mp_token_weights(counts)

            def wts(grp):
                return [host[i] for i in grp]
        for n, grp in enumerate(acc_groups):
            mp.mp_accumulate_group(self.model.plan, [self.gsets[i] for i in grp], wts(grp), n == 0)
        mp.mp_update_step_group(self.model.plan, self.state, [self.gsets[i] for i in fold],
                                wts(fold), not acc_groups, w.max_norm, self.hp)
        return None

    def _step_device_weights(self, s, snapshot):
        """The step with n_i in device memory: the weights from mp_token_weights_dev or, with
        first_counts, computed inside the first accumulation; then the one-micro-batch group
        calls, which read each weight where the kernels run.  first_counts and separate
        together are bench.py's eager step, first_counts alone its captured one."""
        torch, mp, w = self.torch, self.mp, self.w
        plan = self.model.plan
        self.dev_counts = torch.tensor(w.token_counts(s), dtype=torch.int64, device="cuda")
        self.dev_weights = torch.empty(w.k, dtype=torch.float32, device="cuda")
        wp = [self.dev_weights.data_ptr() + 4 * i for i in range(w.k)]
        n_acc = w.k if not self.fold_last else w.k - 1
        in_first = self.first_counts and n_acc >= 1
        if not in_first:
            mp.mp_token_weights_dev(w.k, self.dev_counts, self.dev_weights)
        for i in range(n_acc):
            if i == 0 and in_first:
                mp.mp_accumulate_first_counts(plan, [self.gsets[0]], w.k, self.dev_counts,
                                              self.dev_weights)
            else:
                mp.mp_accumulate_group(plan, [self.gsets[i]], wp[i], i == 0)
        acc_snapshot = ([a.cpu().numpy() for a in self.model.acc]
                        if snapshot and self.model.acc is not None else None)
        if not self.fold_last:
            mp.mp_update_step(plan, self.state, None, 1.0, 0, w.max_norm, self.hp)
        elif self.separate:
            last, lif = [self.gsets[w.k - 1]], w.k == 1
            mp.mp_unscale_check_norm_group(plan, self.state, last, wp[-1], lif, w.max_norm)
            mp.mp_adamw_step_group(plan, self.state, last, wp[-1], lif, self.hp)
            mp.mp_scaler_update(self.state)
        else:
            mp.mp_update_step_group(plan, self.state, [self.gsets[w.k - 1]], wp[-1],
                                    w.k == 1, w.max_norm, self.hp)
        return acc_snapshot

    def host(self, name):
        bufs = getattr(self.model, name)
        out = []
        for b in bufs:
            a = b.cpu()
            if a.dtype in (self.torch.bfloat16, self.torch.float16):
                a = a.view(self.torch.int16).numpy().view(np.uint16)
            else:
                a = a.numpy()
            out.append(a)
        return out

    def close(self):
        for g in self.gsets:
            self.mp.mp_gradset_destroy(g)
        self.mp.mp_state_destroy(self.state)
        self.model.close()


def bits(a):
    """The bit patterns of a float32 or 16-bit array (so NaNs and signed zeros compare exactly)."""
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def compare_state(got, want, prev_master, prev_m, w, same_norm, dt, where=""):
    """Compare one tensor's (or one window's) device state with the oracle's.

    got, want: dicts of "master", "m", "v" (float32) and "w16" (uint16 bit patterns).
    prev_master, prev_m: the oracle's values before the step (for the tolerance bounds).
    same_norm: both sides used the same fp32 norm and clip coefficient, so every value
    must be the same bits; otherwise the parity bar's tolerances apply.
    Returns the number of 16-bit weights that differ from the oracle's; raises
    AssertionError on any violation."""
    # the 16-bit weight is the RNE cast of the device's own master, bit for bit
    assert np.array_equal(got["w16"], oracle.rd16(got["master"], dt)), "w16 != rd16(master)" + where
    if same_norm:
        for nm in ("master", "m", "v", "w16"):
            a, b = bits(got[nm]), bits(want[nm])
            bad = a != b
            if bad.any():
                idx = int(np.flatnonzero(bad)[0])
                raise AssertionError("%s bits differ%s: index %d gpu %r oracle %r"
                                     % (nm, where, idx, got[nm][idx], want[nm][idx]))
        return 0
    # non-finite values carry no rounding: same bits, same places
    for nm in ("master", "m", "v"):
        a, b = got[nm], want[nm]
        fin = np.isfinite(b)
        assert np.array_equal(np.isfinite(a), fin), nm + " non-finite pattern" + where
        assert np.array_equal(bits(a[~fin]), bits(b[~fin])), nm + " non-finite bits" + where
    # tolerance of the parity bar: 2e-6 relative to the magnitude of the terms each
    # value is made of (so cancellation near 0 is judged fairly)
    rtol = 2e-6
    b1 = np.float64(np.float32(w.hp["beta1"]))
    lam = w.hp["lr"] * w.hp["weight_decay"]
    fin = np.isfinite(want["v"])
    r_v = want["v"][fin].astype(np.float64)
    assert rel_within(got["v"][fin], r_v, rtol * np.abs(r_v) + 1e-45).all(), "v tolerance" + where
    fin = np.isfinite(want["m"])
    r_m, m0 = want["m"][fin].astype(np.float64), prev_m[fin].astype(np.float64)
    bound_m = rtol * (b1 * np.abs(m0) + np.abs(r_m - b1 * m0)) + 1e-45
    assert rel_within(got["m"][fin], r_m, bound_m).all(), "m tolerance" + where
    fin = np.isfinite(want["master"])
    r_w, w0 = want["master"][fin].astype(np.float64), prev_master[fin].astype(np.float64)
    bound_w = rtol * (np.abs(w0) * (1 + lam) + np.abs(w0 - r_w)) + 1e-45
    assert rel_within(got["master"][fin], r_w, bound_w).all(), "master tolerance" + where
    # a 16-bit weight may differ only where the two masters differ
    diff16 = bits(got["w16"]) != bits(want["w16"])
    diff32 = bits(got["master"]) != bits(want["master"])
    assert not (diff16 & ~diff32).any(), "w16 differs where the masters agree" + where
    return int(diff16.sum())


def rel_within(x, r, bound):
    """|x - r| <= bound elementwise (all arrays float64)."""
    return np.abs(x.astype(np.float64) - r.astype(np.float64)) <= bound


def compare_step(dev, orc, w, step, acc_dev=None, acc_orc=None):
    """Compare the device state after a step with the oracle's.  Returns a report dict;
    raises AssertionError on any violation of the parity bar."""
    st = dev.stats()
    o = orc.st
    rep = {"step": step, "found_inf": st["found_inf"], "scale": st["scale"],
           "norm_gpu": st["grad_norm"], "norm_oracle": o.norm}
    # integer decisions: bit-exact
    assert st["found_inf"] == int(o.found_inf), rep
    assert st["skipped"] == o.scaler.skipped, rep
    assert st["scale"] == o.scaler.scale, rep
    assert st["good_steps"] == o.scaler.good_steps, rep
    assert st["step"] == o.clock.t, rep
    assert st["skipped_total"] == o.scaler.skipped_total, rep
    assert st["beta1_pow"] == o.clock.p1 and st["beta2_pow"] == o.clock.p2, rep
    if acc_dev is not None:
        for a, b in zip(acc_dev, acc_orc):
            fin = np.isfinite(b)
            assert np.array_equal(a[fin].view(np.uint32), b[fin].view(np.uint32)), "acc bits"
            assert np.array_equal(np.isfinite(a), fin), "acc non-finite pattern"
    if o.found_inf:
        assert not np.isfinite(st["sumsq"]), rep
    else:
        # norm: within 1e-5 relative of the oracle's compensated binary64 value
        # (binary64 sums in two orders: far inside the 1e-5 bar of the norm)
        assert abs(st["sumsq"] - o.sumsq) <= 1e-10 * o.sumsq + 1e-300, rep
        assert abs(st["grad_norm"] - o.norm) <= 1e-5 * o.norm, rep
        assert abs(st["clip_coef"] - o.coef) <= 1e-5 * o.coef, rep
    # a skipped step writes nothing on either side: the state must stay bit-identical
    same_norm = bool(o.found_inf) or (np.float32(st["grad_norm"]) == np.float32(o.norm)
                                      and np.float32(st["clip_coef"]) == np.float32(o.coef))
    rep["same_norm_bits"] = bool(same_norm)
    masters, m, v, w16 = dev.host("master"), dev.host("m"), dev.host("v"), dev.host("w16")
    dt = oracle_dtype(w)
    mism = 0
    for t in range(len(masters)):
        got = {"master": masters[t], "m": m[t], "v": v[t], "w16": w16[t]}
        want = {"master": o.masters[t], "m": o.m[t], "v": o.v[t], "w16": o.w16[t]}
        mism += compare_state(got, want, orc.prev_master[t], orc.prev_m[t], w, same_norm, dt,
                              " (tensor %d)" % t)
    rep["w16_mismatch"] = mism
    return rep


class StreamedOracle:
    """The oracle at full size, streamed: the global norm is recomputed every step from
    regenerated inputs, segment by segment (memory bounded by the segment size), and
    the update itself is computed on sampled windows only.  Each window's fp32 state
    (master, m, v) is carried from step to step by the oracle itself."""

    SEG = 1 << 24

    def __init__(self, w, windows, threads=16, log=print, seg=None):
        self.w, self.windows, self.threads, self.log = w, windows, threads, log
        if seg is not None:
            self.SEG = seg
        self.dt = oracle_dtype(w)
        self.scaler = (oracle.make_scaler(**w.scaler) if w.scaler is not None
                       else oracle.make_scaler(init_scale=1.0, enabled=False))
        self.clock = oracle.make_clock()
        self.state = []
        for t, start, n in windows:
            master = inputs.gen_host_f32(n, w.master_recipe(t), start)
            self.state.append({"master": master, "m": np.zeros(n, np.float32),
                               "v": np.zeros(n, np.float32), "w16": oracle.rd16(master, self.dt)})
        self.segments = [(t, off, min(self.SEG, n - off))
                         for t, n in enumerate(w.numels) for off in range(0, n, self.SEG)]
        self.step_no = 0

    def _grads(self, step, t, start, n, scale):
        w = self.w
        g = [inputs.gen_host_u16(n, w.grad_recipe(step, i, t, scale), w.dtype, start, threads=1)
             for i in range(w.k)]
        inj = w.injection(step)
        if inj is not None and inj[0] == t and start <= inj[1] < start + n:
            g[-1][inj[1] - start] = INF16[w.dtype]
        return g

    def _acc(self, g, weights, n):
        if self.w.k == 1:
            return None
        acc = np.empty(n, np.float32)
        for i in range(self.w.k - 1):
            oracle.accumulate_tensor(g[i], acc, self.dt, weights[i], i == 0)
        return acc

    def step(self):
        from concurrent.futures import ThreadPoolExecutor
        self.step_no += 1
        w, s = self.w, self.step_no
        weights = oracle.token_weights(w.token_counts(s))
        S = self.scaler.scale
        inv = oracle.unscale_factor(S)
        mode = 1 if w.k == 1 else 2
        done = [0]

        def seg_sumsq(seg):
            t, off, n = seg
            g = self._grads(s, t, off, n, S)
            acc = self._acc(g, weights, n)
            r = oracle.unscale_sumsq_tensor(acc, g[-1], n, self.dt, weights[-1], mode, inv)
            done[0] += 1
            if done[0] % 64 == 0:
                self.log("    oracle norm: %d/%d segments" % (done[0], len(self.segments)))
            return r

        with ThreadPoolExecutor(self.threads) as ex:
            parts = list(ex.map(seg_sumsq, self.segments))
        self.found_inf = any(p[0] for p in parts)
        self.sumsq = oracle.sum_in_order([p[1] for p in parts])
        self.norm, self.coef = oracle.norm_and_coef(self.sumsq, self.found_inf, w.max_norm)
        if not self.found_inf:
            b1, b2 = np.float32(w.hp["beta1"]), np.float32(w.hp["beta2"])
            bc1, bc2 = oracle.bias_corrections(self.clock, b1, b2)
            scale = oracle.update_scale(S, self.coef)
            lam = oracle.decay(w.hp["weight_decay"], 1.0)
            for (t, start, n), st in zip(self.windows, self.state):
                st["prev_master"], st["prev_m"] = st["master"].copy(), st["m"].copy()
                g = self._grads(s, t, start, n, S)
                acc = self._acc(g, weights, n)
                oracle.adamw_tensor(acc, g[-1], self.dt, weights[-1], mode, scale, st["master"],
                                    st["m"], st["v"], st["w16"], w.hp["lr"], b1, b2, w.hp["eps"],
                                    lam, bc1, bc2)
            oracle.clock_advance(self.clock, b1, b2)
        oracle.scaler_update(self.scaler, self.found_inf)


def sample_windows(w, per_tensor=512, random_count=64, random_len=4099):
    """First and last `per_tensor` elements of every tensor, plus seeded random windows."""
    wins = []
    for t, n in enumerate(w.numels):
        wins.append((t, 0, min(per_tensor, n)))
        if n > per_tensor:
            lo = max(per_tensor, n - per_tensor)
            wins.append((t, lo, n - lo))
    k = inputs.key(w.cid, inputs.P_SAMPLE)
    big = [t for t, n in enumerate(w.numels) if n > 2 * random_len]
    for i in range(random_count):
        t = big[inputs.draw(k, 2 * i) % len(big)]
        start = inputs.draw(k, 2 * i + 1) % (w.numels[t] - random_len)
        wins.append((t, start, random_len))
    return wins


def compare_windows(dev, so, w):
    """Device state on the sampled windows against the streamed oracle; returns a report."""
    torch = dev.torch
    st = dev.stats()
    rep = {"step": so.step_no, "found_inf": st["found_inf"], "scale": st["scale"],
           "norm_gpu": st["grad_norm"], "norm_oracle": so.norm}
    assert st["found_inf"] == int(so.found_inf), rep
    assert st["scale"] == so.scaler.scale and st["good_steps"] == so.scaler.good_steps, rep
    assert st["skipped"] == so.scaler.skipped, rep
    assert st["step"] == so.clock.t, rep
    assert st["beta1_pow"] == so.clock.p1 and st["beta2_pow"] == so.clock.p2, rep
    if not so.found_inf:
        assert abs(st["sumsq"] - so.sumsq) <= 1e-10 * so.sumsq, rep
        assert abs(st["grad_norm"] - so.norm) <= 1e-5 * so.norm, rep
    same = bool(so.found_inf) or (np.float32(st["grad_norm"]) == np.float32(so.norm)
                                  and np.float32(st["clip_coef"]) == np.float32(so.coef))
    rep["same_norm_bits"] = same
    mism = 0
    for (t, start, n), ost in zip(so.windows, so.state):
        sl = slice(start, start + n)
        got = {"master": dev.model.master[t][sl].cpu().numpy(),
               "m": dev.model.m[t][sl].cpu().numpy(), "v": dev.model.v[t][sl].cpu().numpy(),
               "w16": dev.model.w16[t][sl].cpu().view(torch.int16).numpy().view(np.uint16)}
        if same:
            prev_master = prev_m = None
        else:
            prev_master, prev_m = ost["prev_master"], ost["prev_m"]
        mism += compare_state(got, ost, prev_master, prev_m, w, same, so.dt,
                              " (tensor %d, window at %d)" % (t, start))
    rep["w16_mismatch"] = mism
    rep["windows"] = len(so.windows)
    return rep
