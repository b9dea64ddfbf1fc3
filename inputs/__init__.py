"""Seeded synthetic inputs for the mixed-precision update step.

Serves both the HIP library's tests and benchmark (device fill, ``libmpgen_dev.so``)
and the oracle side (host fill, ``libmpgen_host.so``).  The two fills compile the
same generator header (``mpgen.h``) and give bit-identical arrays.  Nothing here
performs any step of the update itself.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BASE_SEED = 20261202

NORMAL, NORMAL_TAIL, LOGUNIF_MIX, CONST = 0, 1, 2, 3
BF16, FP16 = 0, 1

# stream purposes (the second label of a stream key)
P_MASTER, P_GRAD, P_TOKENS, P_INJECT, P_SIZES, P_SAMPLE = 1, 2, 3, 4, 5, 6


class Recipe(ctypes.Structure):
    _fields_ = [("key", ctypes.c_uint64), ("kind", ctypes.c_int32),
                ("lo_exp", ctypes.c_int32), ("hi_exp", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("sigma", ctypes.c_double),
                ("scale", ctypes.c_double), ("tail_prob", ctypes.c_double),
                ("tail_mult", ctypes.c_double)]


def recipe(key, kind=NORMAL, sigma=1.0, scale=1.0, tail_prob=0.0, tail_mult=1.0, lo_exp=0,
           hi_exp=1):
    return Recipe(key=key, kind=kind, lo_exp=lo_exp, hi_exp=hi_exp, pad=0, sigma=sigma,
                  scale=scale, tail_prob=tail_prob, tail_mult=tail_mult)


_host = None
_dev = None


def host():
    global _host
    if _host is None:
        if not os.path.exists(_build.HOST_LIB):
            _build.build_host()
        L = ctypes.CDLL(_build.HOST_LIB)
        u64, i64, P = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        L.mpgen_fill_f32_host.argtypes = [P, i64, i64, ctypes.POINTER(Recipe), ctypes.c_int]
        L.mpgen_fill_u16_host.argtypes = [P, i64, i64, ctypes.POINTER(Recipe), ctypes.c_int,
                                          ctypes.c_int]
        L.mpgen_key_host.argtypes = [u64] * 5
        L.mpgen_key_host.restype = u64
        L.mpgen_draw_host.argtypes = [u64, u64]
        L.mpgen_draw_host.restype = u64
        L.mpgen_uniform_host.argtypes = [u64, u64]
        L.mpgen_uniform_host.restype = ctypes.c_double
        _host = L
    return _host


def dev():
    """Device twin; loaded after torch so both share torch's HIP runtime."""
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (HIP runtime comes from torch's process image)
        if not os.path.exists(_build.DEV_LIB):
            raise RuntimeError("libmpgen_dev.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_build.DEV_LIB)
        i64, P = ctypes.c_int64, ctypes.c_void_p
        L.mpgen_fill_f32_dev.argtypes = [P, i64, i64, ctypes.POINTER(Recipe), P]
        L.mpgen_fill_f32_dev.restype = ctypes.c_int
        L.mpgen_fill_u16_dev.argtypes = [P, i64, i64, ctypes.POINTER(Recipe), ctypes.c_int, P]
        L.mpgen_fill_u16_dev.restype = ctypes.c_int
        _dev = L
    return _dev


def key(*labels, seed=BASE_SEED):
    labels = list(labels) + [0] * (4 - len(labels))
    assert len(labels) == 4
    return host().mpgen_key_host(seed, *[int(x) & (2 ** 64 - 1) for x in labels])


def draw(k, index):
    return host().mpgen_draw_host(k, index)


def uniform(k, index):
    return host().mpgen_uniform_host(k, index)


def fill_host_f32(out, r, offset=0, threads=0):
    """Elements offset .. offset+n-1 of stream r (threads: 0 = OpenMP default, 1 = caller only)."""
    assert out.dtype == np.float32 and out.flags.c_contiguous
    host().mpgen_fill_f32_host(out.ctypes.data, out.size, offset, ctypes.byref(r), threads)
    return out


def fill_host_u16(out, r, dtype, offset=0, threads=0):
    assert out.dtype == np.uint16 and out.flags.c_contiguous
    host().mpgen_fill_u16_host(out.ctypes.data, out.size, offset, ctypes.byref(r), dtype, threads)
    return out


def gen_host_f32(n, r, offset=0, threads=0):
    return fill_host_f32(np.empty(n, np.float32), r, offset, threads)


def gen_host_u16(n, r, dtype, offset=0, threads=0):
    return fill_host_u16(np.empty(n, np.uint16), r, dtype, offset, threads)


def fill_dev_f32(t, r, offset=0, stream=None):
    import torch
    assert t.dtype == torch.float32 and t.is_cuda and t.is_contiguous()
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = dev().mpgen_fill_f32_dev(t.data_ptr(), t.numel(), offset, ctypes.byref(r), s)
    if rc != 0:
        raise RuntimeError("device fill failed: %d" % rc)
    return t


def fill_dev_u16(t, r, dtype, offset=0, stream=None):
    import torch
    assert t.element_size() == 2 and t.is_cuda and t.is_contiguous()
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = dev().mpgen_fill_u16_dev(t.data_ptr(), t.numel(), offset, ctypes.byref(r), dtype, s)
    if rc != 0:
        raise RuntimeError("device fill failed: %d" % rc)
    return t
