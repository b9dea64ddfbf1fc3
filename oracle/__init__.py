"""Oracle for the mixed-precision update step -- TEST INFRASTRUCTURE ONLY.

A ctypes binding over ``libmporacle.so`` (plain C99 scalar loops, built by
``oracle/build.py``), plus ``OracleStep``, which strings the per-tensor
functions together in the order the pages give for one logical update.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never does.

Every function states the passage it follows; the C source carries the full
citations.  Page titles used below:

* "Mixed precision, loss scaling, gradient accumulation, and activation
  checkpointing" -- called [MP].
* "Megatron Internals III: Mixed Precision, Loss Scaling, and Grad Clipping"
  -- [MEG].
* "Your weights fit on one device but Adam's moments do not" -- [ZQ].
* "Accumulate gradients and recompute activations" -- [RS].
* "Chapter 41 Training at Scale" -- [TS].
"""
import ctypes
import os

import numpy as np

from . import build as _build

BF16 = 0
FP16 = 1

_lib = None


def lib(path=None):
    """Load the oracle library, building it first if it is not built yet."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = _bind(ctypes.CDLL(_build.LIB))
    return _lib


class AdamClock(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int64), ("p1", ctypes.c_double), ("p2", ctypes.c_double)]


class Scaler(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("good_steps", ctypes.c_int32),
                ("growth", ctypes.c_float), ("backoff", ctypes.c_float),
                ("min_scale", ctypes.c_float), ("max_scale", ctypes.c_float),
                ("interval", ctypes.c_int32), ("enabled", ctypes.c_int32),
                ("skipped", ctypes.c_int32), ("skipped_total", ctypes.c_int64)]


_P = ctypes.c_void_p


def _bind(L):
    i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
    L.or_rd16.argtypes = [f32, i32]
    L.or_rd16.restype = ctypes.c_uint16
    L.or_widen16.argtypes = [ctypes.c_uint16, i32]
    L.or_widen16.restype = f32
    L.or_rd16_array.argtypes = [_P, _P, i64, i32]
    L.or_widen16_array.argtypes = [_P, _P, i64, i32]
    L.or_token_weights.argtypes = [i32, _P, _P]
    L.or_token_weights.restype = i32
    L.or_accumulate_tensor.argtypes = [_P, _P, i64, i32, f32, i32]
    L.or_unscale_sumsq_tensor.argtypes = [_P, _P, i64, i32, f32, i32, f32, _P]
    L.or_unscale_sumsq_tensor.restype = i32
    L.or_sum_in_order.argtypes = [_P, i64]
    L.or_sum_in_order.restype = f64
    L.or_norm_and_coef.argtypes = [f64, i32, f32, _P, _P]
    L.or_bias_corrections.argtypes = [_P, f32, f32, _P, _P]
    L.or_clock_advance.argtypes = [_P, f32, f32]
    L.or_adamw_tensor.argtypes = [_P, _P, i64, i32, f32, i32, f32, _P, _P, _P, _P,
                                  f32, f32, f32, f32, f32, f32, f32]
    L.or_scaler_update.argtypes = [_P, i32]
    L.or_unscale_factor.argtypes = [f32]
    L.or_unscale_factor.restype = f32
    L.or_update_scale.argtypes = [f32, f32]
    L.or_update_scale.restype = f32
    L.or_decay.argtypes = [f32, f32]
    L.or_decay.restype = f32
    L.or_e4m3.argtypes = [f32]
    L.or_e4m3.restype = ctypes.c_uint8
    L.or_e4m3_array.argtypes = [_P, _P, i64]
    L.or_e4m3_value.argtypes = [ctypes.c_uint8]
    L.or_e4m3_value.restype = f32
    L.or_fp8_block_cast.argtypes = [_P, i64, i32, _P, _P]
    L.or_fp8_block_cast.restype = i32
    L.or_model_state_bytes.argtypes = [i64]
    L.or_model_state_bytes.restype = i64
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(a, dtype, n=None):
    assert isinstance(a, np.ndarray) and a.dtype == dtype and a.flags.c_contiguous, (
        "oracle arrays must be C-contiguous numpy arrays of %s" % dtype)
    if n is not None:
        assert a.size == n


# --- 16-bit formats ([MP] section 2 "Two 16-bit formats") -------------------

def rd16(x, dtype, L=None):
    """RNE rounding of fp32 values into bf16/fp16 bit patterns (uint16)."""
    L = L or lib()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    L.or_rd16_array(_ptr(x), _ptr(out), x.size, dtype)
    return out


def widen16(h, dtype, L=None):
    """Exact fp32 values of bf16/fp16 bit patterns."""
    L = L or lib()
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    L.or_widen16_array(_ptr(h), _ptr(out), h.size, dtype)
    return out


# --- token weights ([RS] "Weight each mean by the targets it represents") ---

def token_weights(counts, L=None):
    """w_i = fp32(n_i / N) with N = sum n_i; raises ValueError when refused."""
    L = L or lib()
    n = np.ascontiguousarray(counts, dtype=np.int64)
    w = np.empty(n.size, dtype=np.float32)
    if L.or_token_weights(n.size, _ptr(n), _ptr(w)) != 0:
        raise ValueError("token counts refused: every n_i must be > 0 and N <= 2^53")
    return w


# --- per-tensor steps --------------------------------------------------------

def accumulate_tensor(g16, acc, dtype, w, first, L=None):
    """acc = w*widen(g16) (first) or acc + w*widen(g16) ([MP] "Gradient accumulation")."""
    L = L or lib()
    _check(g16, np.uint16)
    _check(acc, np.float32, g16.size)
    L.or_accumulate_tensor(_ptr(g16), _ptr(acc), g16.size, dtype, float(w), int(bool(first)))


def unscale_sumsq_tensor(acc, g16_last, n, dtype, w_last, mode, inv_scale, L=None):
    """(found_inf, sum of squares) of g = g_eff / S ([MEG] sections 4 and 9)."""
    L = L or lib()
    if acc is not None:
        _check(acc, np.float32, n)
    if g16_last is not None:
        _check(g16_last, np.uint16, n)
    out = ctypes.c_double()
    fi = L.or_unscale_sumsq_tensor(_ptr(acc), _ptr(g16_last), n, dtype, float(w_last),
                                   mode, float(inv_scale), ctypes.byref(out))
    return bool(fi), out.value


def unscale_factor(scale, L=None):
    """1/S ([MP] "Loss scaling")."""
    return (L or lib()).or_unscale_factor(float(scale))


def update_scale(scale, coef, L=None):
    """(1/S) * coef, the factor AdamW applies to each fp32 gradient ([MEG] section 9)."""
    return (L or lib()).or_update_scale(float(scale), float(coef))


def decay(weight_decay, multiplier, L=None):
    return (L or lib()).or_decay(float(weight_decay), float(multiplier))


def sum_in_order(parts, L=None):
    L = L or lib()
    p = np.ascontiguousarray(parts, dtype=np.float64)
    return L.or_sum_in_order(_ptr(p), p.size)


def norm_and_coef(sumsq, found_inf, max_norm, L=None):
    """(norm, coef) with coef = min(1, max_norm/(norm+1e-6)) ([MEG] section 9)."""
    L = L or lib()
    norm, coef = ctypes.c_float(), ctypes.c_float()
    L.or_norm_and_coef(float(sumsq), int(bool(found_inf)), float(max_norm),
                       ctypes.byref(norm), ctypes.byref(coef))
    return norm.value, coef.value


def bias_corrections(clock, beta1, beta2, L=None):
    L = L or lib()
    b1, b2 = ctypes.c_float(), ctypes.c_float()
    L.or_bias_corrections(ctypes.byref(clock), float(beta1), float(beta2),
                          ctypes.byref(b1), ctypes.byref(b2))
    return b1.value, b2.value


def clock_advance(clock, beta1, beta2, L=None):
    L = L or lib()
    L.or_clock_advance(ctypes.byref(clock), float(beta1), float(beta2))


def adamw_tensor(acc, g16_last, dtype, w_last, mode, scale, master, m, v, w16,
                 lr, beta1, beta2, eps, lam, bc1, bc2, L=None):
    """AdamW + RNE cast on one tensor, in place ([ZQ]; [RS]; [MP] section 2)."""
    L = L or lib()
    n = master.size
    for a, t in ((master, np.float32), (m, np.float32), (v, np.float32), (w16, np.uint16)):
        _check(a, t, n)
    if acc is not None:
        _check(acc, np.float32, n)
    if g16_last is not None:
        _check(g16_last, np.uint16, n)
    L.or_adamw_tensor(_ptr(acc), _ptr(g16_last), n, dtype, float(w_last), mode, float(scale),
                      _ptr(master), _ptr(m), _ptr(v), _ptr(w16),
                      float(lr), float(beta1), float(beta2), float(eps), float(lam),
                      float(bc1), float(bc2))


def scaler_update(scaler, found_inf, L=None):
    """Dynamic loss-scale controller ([MP] "Dynamic scaling"; [MEG] section 5)."""
    L = L or lib()
    L.or_scaler_update(ctypes.byref(scaler), int(bool(found_inf)))


def model_state_bytes(params, L=None):
    """2 + 2 + 4 + 4 + 4 bytes per parameter ([TS] equation (41.1))."""
    L = L or lib()
    return L.or_model_state_bytes(int(params))


def e4m3(x, L=None):
    """E4M3 codes of fp32 values (RNE, saturating at 448) ([TS] section 41.5)."""
    L = L or lib()
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.size, np.uint8)
    L.or_e4m3_array(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_value(codes, L=None):
    L = L or lib()
    return np.array([L.or_e4m3_value(int(c)) for c in np.asarray(codes).ravel()], np.float32)


def fp8_block_cast(x, block=16, L=None):
    """(codes, scales) of the fine-grained FP8 cast ([TS] section 41.5, listing 41.5)."""
    L = L or lib()
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    if block <= 0 or x.size % block:
        raise ValueError("the length must be divisible by block")
    codes = np.empty(x.size, np.uint8)
    scales = np.empty(x.size // block, np.float32)
    if L.or_fp8_block_cast(_ptr(x), x.size, block, _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("the length must be divisible by block")
    return codes, scales


def make_scaler(init_scale=2.0 ** 16, growth=2.0, backoff=0.5, min_scale=1.0,
                max_scale=2.0 ** 64, interval=2000, enabled=True):
    return Scaler(scale=init_scale, good_steps=0, growth=growth, backoff=backoff,
                  min_scale=min_scale, max_scale=max_scale, interval=interval,
                  enabled=int(bool(enabled)), skipped=0, skipped_total=0)


def make_clock():
    return AdamClock(t=0, p1=1.0, p2=1.0)


from .step import OracleStep  # noqa: E402,F401
