"""Mutation check of the oracle's pins (CPU only).

Each mutant plants one plausible mistake in a copy of the oracle -- the pitfalls
listed in section 5 of "Mixed precision, loss scaling, gradient accumulation,
and activation checkpointing" plus dropped terms, wrong signs and swapped
operands in the update -- and the pins in test_oracle_pins.py must reject it.
The mistake is planted in a temporary copy on the CPU; the real oracle is never
modified.
"""
import importlib.util
import inspect
import os
import shutil
import sys

import pytest

import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C = "mpstep_oracle.c"
STEP = "step.py"

# (id, file, original text, mutated text)
MUTANTS = [
    ("rd16-truncates", C, "double r = nearbyint(X / quantum);", "double r = trunc(X / quantum);"),
    ("rd16-ties-away", C, "double r = nearbyint(X / quantum);", "double r = round(X / quantum);"),
    ("rd16-no-overflow", C, "if (fabs(Y) > or_max_finite(f)) Y = negative ? -INFINITY : INFINITY;",
     ""),
    ("rd16-nan-not-quiet", C, "| emask | quiet);", "| emask);"),
    ("widen-subnormal-exponent", C, "v = ldexp((double)M, 1 - f.bias - mbits);",
     "v = ldexp((double)M, -f.bias - mbits);"),
    ("weights-one-over-k (pitfall 7)", C, "w[i] = (float)((double)n[i] / (double)total);",
     "w[i] = (float)(1.0 / (double)k);"),
    ("weights-summed (pitfall 8)", C, "w[i] = (float)((double)n[i] / (double)total);",
     "w[i] = 1.0f;"),
    ("zero-count-accepted", C, "if (n[i] <= 0) return -1;", "if (n[i] < 0) return -1;"),
    ("total-limit-off-by-one", C, "if (n[i] > ((int64_t)1 << 53) - total) return -1;",
     "if (n[i] > ((int64_t)1 << 53) - total + 1) return -1;"),
    ("zeroing-between-microbatches (pitfall 9)", C, "else       acc[j] = acc[j] + contribution;",
     "else       acc[j] = contribution;"),
    ("first-ignored-keeps-bad-grads (pitfall 13)", C, "if (first) acc[j] = contribution;",
     "if (0) acc[j] = contribution;"),
    ("weight-not-applied", C, "float contribution = w * a;", "float contribution = a;"),
    ("fold-drops-accumulator", C, "return acc[j] + contribution;", "return contribution;"),
    ("never-unscale-in-norm (pitfall 11/15)", C,
     "float g = or_effective_grad(acc, g16, j, dtype, w_last, mode) * inv_scale;",
     "float g = or_effective_grad(acc, g16, j, dtype, w_last, mode);"),
    ("unscale-multiplies-by-S", C, "return 1.0f / scale;\n}\n\n/* The factor",
     "return scale;\n}\n\n/* The factor"),
    ("never-unscale-in-update (pitfall 11)", C, "return (1.0f / scale) * coef;", "return coef;"),
    ("clip-not-applied", C, "return (1.0f / scale) * coef;", "return (1.0f / scale);"),
    ("overflow-not-flagged (pitfall 12)", C, "if (!isfinite(g)) found_inf = 1;", ""),
    ("no-compensation", C, "return isfinite(k->sum) ? k->sum + k->comp : k->sum;",
     "return k->sum;"),
    ("norm-without-sqrt", C, "float norm = (float)sqrt(sumsq);", "float norm = (float)sumsq;"),
    ("clip-when-below-limit", C, "coef = q < 1.0f ? q : 1.0f;", "coef = q;"),
    ("clip-on-overflowed-step", C, "if (max_norm > 0.0f && !found_inf) {",
     "if (max_norm > 0.0f) {"),
    ("clip-inverted", C, "float q = max_norm / (norm + 1e-6f);",
     "float q = (norm + 1e-6f) / max_norm;"),
    ("bias-correction-beta-not-power", C, "double p1 = c->p1 * (double)beta1;",
     "double p1 = (double)beta1;"),
    ("no-bias-correction-m", C, "float mh = mj / bc1;", "float mh = mj;"),
    ("no-bias-correction-v", C, "float vh = vj / bc2;", "float vh = vj;"),
    ("beta1-beta2-swapped", C, "float mj = beta1 * m[j] + ob1 * gs;",
     "float mj = beta2 * m[j] + ob1 * gs;"),
    ("v-linear-in-g", C, "float vj = beta2 * v[j] + ob2 * (gs * gs);",
     "float vj = beta2 * v[j] + ob2 * gs;"),
    ("m-momentum-dropped", C, "float mj = beta1 * m[j] + ob1 * gs;", "float mj = ob1 * gs;"),
    ("eps-inside-sqrt", C, "float den = sqrtf(vh) + eps;", "float den = sqrtf(vh + eps);"),
    ("no-sqrt", C, "float den = sqrtf(vh) + eps;", "float den = vh + eps;"),
    ("update-sign", C, "w = w - lr * (u + lambda * w);", "w = w + lr * (u + lambda * w);"),
    ("decay-sign", C, "w = w - lr * (u + lambda * w);", "w = w - lr * (u - lambda * w);"),
    ("decay-dropped", C, "w = w - lr * (u + lambda * w);", "w = w - lr * u;"),
    ("decay-not-scaled-by-lr", C, "w = w - lr * (u + lambda * w);",
     "w = w - lr * u - lambda * w;"),
    ("cast-from-old-master", C, "master[j] = w;\n        w16[j] = or_rd16(w, dtype);",
     "w16[j] = or_rd16(master[j], dtype);\n        master[j] = w;"),
    ("decay-multiplier-ignored", C, "return weight_decay * multiplier;", "return weight_decay;"),
    ("count-not-restarted (pitfall 14)", C,
     "s->scale = next > s->min_scale ? next : s->min_scale;\n        s->good_steps = 0;",
     "s->scale = next > s->min_scale ? next : s->min_scale;"),
    ("growth-off-by-one", C, "if (s->good_steps == s->interval) {",
     "if (s->good_steps + 1 == s->interval) {"),
    ("backoff-divides", C, "float next = s->scale * s->backoff;",
     "float next = s->scale / s->backoff;"),
    ("no-min-scale", C, "s->scale = next > s->min_scale ? next : s->min_scale;",
     "s->scale = next;"),
    ("no-max-scale", C, "s->scale = next < s->max_scale ? next : s->max_scale;",
     "s->scale = next;"),
    ("growth-count-not-restarted", C,
     "s->scale = next < s->max_scale ? next : s->max_scale;\n            s->good_steps = 0;",
     "s->scale = next < s->max_scale ? next : s->max_scale;"),
    ("scaler-ignores-enabled", C, "if (!s->enabled) return;", ""),
    ("skip-not-recorded", C, "s->skipped = found_inf ? 1 : 0;", "s->skipped = 0;"),
    ("accounting-drops-grad", C, "return params * (2 + 2 + 4 + 4 + 4);",
     "return params * (2 + 4 + 4 + 4);"),
    ("fp8-scale-without-abs", C, "float a = fabsf(xb[i]);", "float a = xb[i];"),
    ("fp8-zero-block-scale", C, "if (scale == 0.0f) scale = 1.0f;", ""),
    ("fp8-multiplies-by-scale", C, "float q = x / scale;", "float q = x * scale;"),
    ("fp8-scale-wrong-max", C, "float scale = amax / 448.0f;", "float scale = amax / 480.0f;"),
    ("fp8-max-ignores-nan", C, "if (isnan(a) || a > amax) amax = a;", "if (a > amax) amax = a;"),
    ("fp8-nan-quotient-sign-from-machine", C, "if (isnan(q)) q = copysignf(NAN, x);", ""),
    ("e4m3-truncates", C, "Y = nearbyint(X / quantum) * quantum;", "Y = trunc(X / quantum) * quantum;"),
    ("e4m3-bias", C, "return (uint8_t)(sign | (uint32_t)((e + 7) << 3) | mant);",
     "return (uint8_t)(sign | (uint32_t)((e + 8) << 3) | mant);"),
    ("e4m3-subnormal-quantum", C, "if (e < -6) e = -6;                       /* subnormal",
     "if (e < -7) e = -7;                       /* subnormal"),
    ("e4m3-no-saturation", C, "if (Y > 448.0) Y = 448.0;                 /* saturate */", ""),
    ("step-on-overflow (pitfall 12)", STEP, "        if self.found_inf:\n            return False\n",
     ""),
    ("clock-not-advanced", STEP, "        clock_advance(self.clock, beta1, beta2, self.L)\n", ""),
    ("clock-advanced-on-skip", STEP, "        if self.found_inf:\n            return False\n",
     "        if self.found_inf:\n            clock_advance(self.clock, beta1, beta2, self.L)\n"
     "            return False\n"),
    ("norm-only-last-tensor", STEP, "self.sumsq = sum_in_order([p[1] for p in parts], self.L)",
     "self.sumsq = parts[-1][1]"),
    ("inf-only-first-tensor", STEP, "self.found_inf = any(p[0] for p in parts)",
     "self.found_inf = parts[0][0]"),
]


def _pin_tests():
    """Pin functions, cheapest first (the rd16 comparisons over 2M patterns go last)."""
    fns = [f for n, f in inspect.getmembers(pins, inspect.isfunction)
           if n.startswith("test_") and "exhaustive" not in n]
    slow = {"test_rd16_fp16_vs_numpy", "test_rd16_bf16_vs_torch"}
    return sorted(fns, key=lambda f: (f.__name__ in slow, f.__code__.co_firstlineno))


def _load_mutant(tmp, idx, fname, old, new):
    pkg = "oracle_mutant_%d" % idx
    d = os.path.join(tmp, pkg)
    shutil.copytree(os.path.join(ROOT, "oracle"), d,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp"))
    path = os.path.join(d, fname)
    src = open(path).read()
    assert src.count(old) == 1, "mutation site not unique or missing: %r" % old
    open(path, "w").write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(pkg, os.path.join(d, "__init__.py"),
                                                  submodule_search_locations=[d])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[pkg] = mod
    spec.loader.exec_module(mod)
    mod._build.build()
    return mod


@pytest.mark.parametrize("idx", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_pins_kill_mutant(idx, tmp_path, monkeypatch):
    name, fname, old, new = MUTANTS[idx]
    mod = _load_mutant(str(tmp_path), idx, fname, old, new)
    monkeypatch.setattr(pins, "oracle", mod)
    L = mod.lib()
    killed_by = None
    for fn in _pin_tests():
        kwargs = {"orc": L} if "orc" in inspect.signature(fn).parameters else {}
        try:
            fn(**kwargs)
        except (Exception, pytest.fail.Exception):  # noqa: BLE001 -- any failed pin kills it
            killed_by = fn.__name__
            break
    assert killed_by is not None, "mutant %r survived every pin" % name
