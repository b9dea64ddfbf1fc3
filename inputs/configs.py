"""Synthetic workloads shaped like the pages' training runs.

Each workload is a list of named parameter tensors with the shapes of a model
family, plus the recipe of every input the update step reads: fp32 masters,
per-micro-batch 16-bit gradients, token counts and (for the fp16 run) an
injected overflow.  Every value comes from the counter-based generator in
``mpgen.h``, keyed by (workload id, purpose, step, micro-batch, tensor), so any
element can be regenerated on its own, on the host or on the device.

Workloads (ids are stream labels):

* 1  ``llama-10.5M``  d=256, 8 layers, ffn 688, vocab 8192, untied head; bf16, k=4
* 2  ``gpt-124M``     d=768, 12 layers, vocab 50304, context 1024, tied; fp16, k=1,
  dynamic loss scale from 2^16, +inf injected on step 3
* 3  ``gpt-1.3B``     d=2048, 24 layers, ffn 8192, vocab 50304, context 2048, tied; bf16, k=8,
  N(0, 1e-4) gradients with a 1e-3 fraction scaled by 100
* 4  ``ragged-4096``  4096 tensors, 4092 log-uniform sizes + {64, 65, 2^24-1, 2^24}; bf16, k=4
* 5  ``llama3-8B``    d=4096, 32 layers, GQA kv 1024, ffn 14336, vocab 128256 untied; bf16, k=4
* 13, 14, 15: reduced versions of 3, 4 and 5 for element-by-element parity;
  16, 17, 19: lists of edge-case sizes around the kernels' tile boundaries (bf16; fp16 with
  a dynamic scale and an injected overflow; the same on sizes that are multiples of 16);
  18: the fp16 run's scaler over 2003 steps on three small tensors;
  20: one tensor of 2^31 + 4097 elements and one of 7.
"""
import math

from . import (key, draw, uniform, recipe, NORMAL, NORMAL_TAIL, LOGUNIF_MIX, BF16, FP16,
               P_MASTER, P_GRAD, P_TOKENS, P_INJECT, P_SIZES)


def llama_tensors(d, layers, ffn, vocab, kv=None):
    kv = kv or d
    ts = [("tok_embed", (vocab, d))]
    for i in range(layers):
        p = "layers.%d." % i
        ts += [(p + "attn_norm", (d,)), (p + "wq", (d, d)), (p + "wk", (kv, d)),
               (p + "wv", (kv, d)), (p + "wo", (d, d)), (p + "ffn_norm", (d,)),
               (p + "w_gate", (ffn, d)), (p + "w_up", (ffn, d)), (p + "w_down", (d, ffn))]
    ts += [("final_norm", (d,)), ("lm_head", (vocab, d))]
    return ts


def gpt_tensors(d, layers, ffn, vocab, ctx):
    ts = [("wte", (vocab, d)), ("wpe", (ctx, d))]
    for i in range(layers):
        p = "h.%d." % i
        ts += [(p + "ln1.w", (d,)), (p + "ln1.b", (d,)), (p + "qkv.w", (3 * d, d)),
               (p + "qkv.b", (3 * d,)), (p + "proj.w", (d, d)), (p + "proj.b", (d,)),
               (p + "ln2.w", (d,)), (p + "ln2.b", (d,)), (p + "fc.w", (ffn, d)),
               (p + "fc.b", (ffn,)), (p + "mproj.w", (d, ffn)), (p + "mproj.b", (d,))]
    ts += [("lnf.w", (d,)), ("lnf.b", (d,))]
    return ts


def ragged_tensors(cid, count, lo, ratio, extremes):
    """`count - len(extremes)` sizes round(lo * ratio^U), U uniform on [0, 1), then the extremes."""
    k = key(cid, P_SIZES)
    n_draw = count - len(extremes)
    sizes = [max(1, int(round(lo * math.exp(math.log(ratio) * uniform(k, i)))))
             for i in range(n_draw)]
    sizes += list(extremes)
    return [("t%04d" % i, (n,)) for i, n in enumerate(sizes)]


class Workload:
    def __init__(self, cid, name, tensors, dtype, k, grad_kind=NORMAL, grad_sigma=1e-3,
                 tail_prob=0.0, tail_mult=1.0, lo_exp=0, hi_exp=1, scaler=None,
                 inject_step=None, steps=3, lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8,
                 weight_decay=0.1, max_norm=1.0, master_sigma=0.02):
        self.cid = cid
        self.name = name
        self.tensors = tensors
        self.dtype = dtype
        self.k = k
        self.grad_kind = grad_kind
        self.grad_sigma = grad_sigma
        self.tail_prob = tail_prob
        self.tail_mult = tail_mult
        self.lo_exp, self.hi_exp = lo_exp, hi_exp
        self.scaler = scaler          # None: bf16, no dynamic scale (S = 1)
        self.inject_step = inject_step
        self.steps = steps
        self.hp = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay)
        self.max_norm = max_norm
        self.master_sigma = master_sigma

    @property
    def numels(self):
        return [math.prod(s) for _, s in self.tensors]

    @property
    def total(self):
        return sum(self.numels)

    def master_recipe(self, t):
        return recipe(key(self.cid, P_MASTER, 0, t), NORMAL, sigma=self.master_sigma)

    def grad_recipe(self, step, micro, t, loss_scale=1.0):
        """16-bit gradient of micro-batch `micro` of `step` (1-based), scaled by the loss scale."""
        return recipe(key(self.cid, P_GRAD, step * 1024 + micro, t), self.grad_kind,
                      sigma=self.grad_sigma, scale=loss_scale, tail_prob=self.tail_prob,
                      tail_mult=self.tail_mult, lo_exp=self.lo_exp, hi_exp=self.hi_exp)

    def token_counts(self, step):
        """n_i drawn uniformly from 400..512 (every micro-batch has targets)."""
        if self.k == 1:
            return [451]
        kk = key(self.cid, P_TOKENS, step)
        return [400 + draw(kk, i) % 113 for i in range(self.k)]

    def injection(self, step):
        """(tensor, index) of the +inf planted into the last micro-batch's gradient, or None."""
        if self.inject_step is None or step != self.inject_step:
            return None
        kk = key(self.cid, P_INJECT, step)
        t = draw(kk, 0) % len(self.tensors)
        return t, draw(kk, 1) % self.numels[t]


FP16_SCALER = dict(init_scale=2.0 ** 16, growth=2.0, backoff=0.5, min_scale=1.0,
                   max_scale=2.0 ** 64, interval=2000)


def make(name):
    if name in ("llama-10.5M", "c1"):
        return Workload(1, "llama-10.5M", llama_tensors(256, 8, 688, 8192), BF16, 4)
    if name in ("gpt-124M", "c2"):
        return Workload(2, "gpt-124M", gpt_tensors(768, 12, 3072, 50304, 1024), FP16, 1,
                        grad_kind=LOGUNIF_MIX, tail_prob=0.05, lo_exp=-30, hi_exp=-20,
                        scaler=dict(FP16_SCALER), inject_step=3, steps=5)
    if name in ("gpt-1.3B", "c3"):
        return Workload(3, "gpt-1.3B", gpt_tensors(2048, 24, 8192, 50304, 2048), BF16, 8,
                        grad_kind=NORMAL_TAIL, grad_sigma=1e-4, tail_prob=1e-3, tail_mult=100.0,
                        steps=20)
    if name in ("ragged-4096", "c4"):
        return Workload(4, "ragged-4096",
                        ragged_tensors(4, 4096, 64, 22987.0, [64, 65, 2 ** 24 - 1, 2 ** 24]),
                        BF16, 4)
    if name in ("llama3-8B", "c5"):
        return Workload(5, "llama3-8B", llama_tensors(4096, 32, 14336, 128256, kv=1024), BF16, 4,
                        steps=2)
    if name == "gpt-1.3B-small":
        return Workload(13, name, gpt_tensors(256, 4, 1024, 4096, 256), BF16, 8,
                        grad_kind=NORMAL_TAIL, grad_sigma=1e-4, tail_prob=1e-3, tail_mult=100.0,
                        steps=20)
    if name == "ragged-4096-small":
        return Workload(14, name, ragged_tensors(14, 4096, 1, 4096.0, [1, 65, 2 ** 16 - 1, 2 ** 16]),
                        BF16, 4)
    if name == "llama3-8B-small":
        return Workload(15, name, llama_tensors(512, 2, 1792, 4096, kv=128), BF16, 4, steps=2)
    if name == "edges":
        sizes = [1, 2, 3, 4, 5, 7, 8, 9, 255, 256, 257, 511, 512, 513, 2047, 2048, 2049, 4095,
                 4096, 4097, 65535, 65536, 65537, 1000003]
        return Workload(16, name, [("e%02d" % i, (n,)) for i, n in enumerate(sizes)], BF16, 3)
    if name == "edges-fp16":
        sizes = [1, 3, 8, 9, 2047, 2049, 65537, 300007]
        return Workload(17, name, [("f%02d" % i, (n,)) for i, n in enumerate(sizes)], FP16, 2,
                        grad_kind=LOGUNIF_MIX, tail_prob=0.05, lo_exp=-30, hi_exp=-20,
                        scaler=dict(FP16_SCALER, interval=2), inject_step=2, steps=6)
    if name == "edges-fp16-b16":
        # the fp16 edge list's recipe, scaler and overflow on sizes that are mostly multiples of
        # 16 around the tile boundaries (for the fused block-16 FP8 cast), plus three that are not
        sizes = [16, 32, 48, 2032, 2048, 2064, 4112, 65536, 1, 9, 300007]
        return Workload(19, name, [("b%02d" % i, (n,)) for i, n in enumerate(sizes)], FP16, 2,
                        grad_kind=LOGUNIF_MIX, tail_prob=0.05, lo_exp=-30, hi_exp=-20,
                        scaler=dict(FP16_SCALER, interval=2), inject_step=2, steps=5)
    if name == "huge-tensor":
        # one tensor past 2^31 elements (element offsets that need 64 bits everywhere: chunk
        # starts, pointers, generator indices) next to a tiny one; bf16, k = 2
        return Workload(20, name, [("big", (2 ** 31 + 4097,)), ("small", (7,))], BF16, 2, steps=2)
    if name == "edges-k1":
        # the bf16 edge list with one micro-batch: no accumulator, so the norm reads the 16-bit
        # gradient alone and its blocks each walk several ragged chunks
        sizes = [1, 2, 3, 4, 5, 7, 8, 9, 255, 256, 257, 511, 512, 513, 2047, 2048, 2049, 4095,
                 4096, 4097, 65535, 65536, 65537, 1000003]
        return Workload(21, name, [("k%02d" % i, (n,)) for i, n in enumerate(sizes)], BF16, 1)
    if name == "gpt-124M-scaler":
        # the fp16 run's scaler, overflow and gradient recipe on a small tensor list, long enough
        # for the scale to grow back: 2000 clean steps after the overflow of step 3
        return Workload(18, name, [("a", (1000,)), ("b", (3001,)), ("c", (768,))], FP16, 1,
                        grad_kind=LOGUNIF_MIX, tail_prob=0.05, lo_exp=-30, hi_exp=-20,
                        scaler=dict(FP16_SCALER), inject_step=3, steps=2003)
    raise KeyError(name)


FULL = ["llama-10.5M", "gpt-124M", "gpt-1.3B", "ragged-4096", "llama3-8B"]
