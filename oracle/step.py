"""One logical update over a list of tensors, on host arrays -- TEST INFRASTRUCTURE ONLY.

The order is the one the pages give for a mixed-precision optimizer step
("Megatron Internals III", section 9, order of operations; "Accumulate gradients
and recompute activations", "Weight each mean by the targets it represents"):

1. accumulate the k token-weighted micro-batch gradients into fp32 buffers;
2. unscale by 1/S and check every value for inf/NaN;
3. global L2 norm over all tensors, clip coefficient;
4. unless the check failed: AdamW on the fp32 masters and moments, then the
   RNE cast of the masters back to the 16-bit model weights;
5. the loss-scaler decision.

The per-element arithmetic lives in ``mpstep_oracle.c``.  Python only loops
over tensors.  Optional threads split the work by tensor; the per-tensor sums
of squares are still combined in tensor order, so the result does not depend
on the thread count.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import (accumulate_tensor, unscale_sumsq_tensor, sum_in_order, norm_and_coef,
               bias_corrections, clock_advance, adamw_tensor, scaler_update,
               unscale_factor, update_scale, decay, make_scaler, make_clock, lib)


class OracleStep:
    """Host-side model state: fp32 masters, m, v, 16-bit weights, fp32 accumulators."""

    def __init__(self, dtype, masters, w16, m=None, v=None, wd_mult=None, scaler=None,
                 clock=None, with_acc=True, threads=1):
        self.dtype = dtype
        self.masters = masters
        self.w16 = w16
        self.m = m if m is not None else [np.zeros_like(x) for x in masters]
        self.v = v if v is not None else [np.zeros_like(x) for x in masters]
        self.acc = [np.zeros_like(x) for x in masters] if with_acc else None
        self.wd_mult = wd_mult if wd_mult is not None else [1.0] * len(masters)
        self.scaler = scaler if scaler is not None else make_scaler(enabled=False, init_scale=1.0)
        self.clock = clock if clock is not None else make_clock()
        self.threads = threads
        self.found_inf = False
        self.sumsq = 0.0
        self.norm = 0.0
        self.coef = 1.0
        self.L = lib()

    def _map(self, fn, n):
        if self.threads <= 1:
            return [fn(i) for i in range(n)]
        with ThreadPoolExecutor(self.threads) as ex:
            return list(ex.map(fn, range(n)))

    @property
    def numels(self):
        return [x.size for x in self.masters]

    def accumulate(self, g16, weight, first):
        """acc_t = w*g16_t (first) or acc_t + w*g16_t for every tensor t."""
        assert self.acc is not None, "this state was built without accumulators"
        self._map(lambda i: accumulate_tensor(g16[i], self.acc[i], self.dtype, weight, first,
                                              self.L), len(self.masters))

    def _mode(self, g16_last, last_is_first):
        if g16_last is None:
            return 0
        return 1 if last_is_first else 2

    def unscale_check_norm(self, g16_last=None, w_last=1.0, last_is_first=False, max_norm=0.0):
        """found_inf, sum of squares, norm and clip coefficient of the unscaled gradient."""
        mode = self._mode(g16_last, last_is_first)
        inv_scale = unscale_factor(self.scaler.scale, self.L)

        def one(i):
            acc = None if (self.acc is None or mode == 1) else self.acc[i]
            g = None if g16_last is None else g16_last[i]
            return unscale_sumsq_tensor(acc, g, self.masters[i].size, self.dtype, w_last, mode,
                                        inv_scale, self.L)

        parts = self._map(one, len(self.masters))
        self.found_inf = any(p[0] for p in parts)
        self.sumsq = sum_in_order([p[1] for p in parts], self.L)
        self.norm, self.coef = norm_and_coef(self.sumsq, self.found_inf, max_norm, self.L)
        return self.found_inf, self.sumsq, self.norm, self.coef

    def adamw_step(self, g16_last=None, w_last=1.0, last_is_first=False, lr=3e-4, beta1=0.9,
                   beta2=0.95, eps=1e-8, weight_decay=0.1):
        """AdamW + cast on every tensor; nothing changes when the check failed."""
        if self.found_inf:
            return False
        mode = self._mode(g16_last, last_is_first)
        beta1, beta2 = np.float32(beta1), np.float32(beta2)
        bc1, bc2 = bias_corrections(self.clock, beta1, beta2, self.L)
        scale = update_scale(self.scaler.scale, self.coef, self.L)

        def one(i):
            acc = None if (self.acc is None or mode == 1) else self.acc[i]
            g = None if g16_last is None else g16_last[i]
            lam = decay(weight_decay, self.wd_mult[i], self.L)
            adamw_tensor(acc, g, self.dtype, w_last, mode, scale, self.masters[i], self.m[i],
                         self.v[i], self.w16[i], lr, beta1, beta2, eps, lam, bc1, bc2, self.L)

        self._map(one, len(self.masters))
        clock_advance(self.clock, beta1, beta2, self.L)
        return True

    def scaler_update(self):
        scaler_update(self.scaler, self.found_inf, self.L)
