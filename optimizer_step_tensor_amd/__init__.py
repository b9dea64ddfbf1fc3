"""Python binding of libmpstep, the mixed-precision update step for MI355X.

Argument marshalling only: every entry point forwards to the C ABI declared in
``include/mpstep.h`` (same names, same arguments), and every step of the update
runs in the library's HIP kernels.  PyTorch supplies device memory and streams.
``ModelState`` allocates the buffers of one model with torch and builds the
plan over them; it computes nothing itself.

Importing this module loads ``libmpstep.so``; it raises if the library has not
been built (``python -m optimizer_step_tensor_amd.build`` or
``__graft_entry__.build()``).  There is no fallback implementation.
"""
import ctypes
import os

import torch  # loaded first: libmpstep then binds to torch's HIP runtime

from .build import LIB as _LIB_PATH

MP_BF16 = 0
MP_FP16 = 1

MP_OK, MP_ERR_INVALID, MP_ERR_ALIGN, MP_ERR_NOMEM, MP_ERR_HIP, MP_ERR_ORDER = range(6)

ENTRY_POINTS = [
    "mp_status_string", "mp_last_error", "mp_abi_version", "mp_token_weights",
    "mp_state_bytes_per_param", "mp_plan_create", "mp_plan_destroy", "mp_plan_info",
    "mp_chunk_layout",
    "mp_gradset_create", "mp_gradset_destroy", "mp_state_create", "mp_state_destroy",
    "mp_state_read", "mp_state_scale_ptr", "mp_accumulate", "mp_unscale_check_norm",
    "mp_adamw_step", "mp_scaler_update", "mp_cast_to_16", "mp_widen_16",
    "mp_state_export", "mp_state_import", "mp_norm_partial", "mp_norm_finish",
    "mp_cast_fp8_blocks", "mp_fp8set_create", "mp_fp8set_destroy", "mp_adamw_step_fp8",
    "mp_gradset_update", "mp_update_step", "mp_token_weights_dev", "mp_accumulate_group",
    "mp_update_step_group", "mp_unscale_check_norm_group", "mp_adamw_step_group",
    "mp_norm_partial_group", "mp_update_step_noalloc", "mp_accumulate_first_counts",
]

MP_STATE_BLOB_BYTES = 256
MP_NOALLOC_MAX_NORM_BLOCKS = 262144


class MpError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (_name(status), message))
        self.status = status


class ScalerCfg(ctypes.Structure):
    _fields_ = [("init_scale", ctypes.c_float), ("growth", ctypes.c_float),
                ("backoff", ctypes.c_float), ("min_scale", ctypes.c_float),
                ("max_scale", ctypes.c_float), ("interval", ctypes.c_int32),
                ("enabled", ctypes.c_int32)]


class AdamWHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class Stats(ctypes.Structure):
    _fields_ = [("found_inf", ctypes.c_int32), ("skipped", ctypes.c_int32),
                ("good_steps", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("step", ctypes.c_int64), ("skipped_total", ctypes.c_int64),
                ("sumsq", ctypes.c_double), ("beta1_pow", ctypes.c_double),
                ("beta2_pow", ctypes.c_double), ("scale", ctypes.c_float),
                ("grad_norm", ctypes.c_float), ("clip_coef", ctypes.c_float),
                ("reserved1", ctypes.c_float)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_
                if not name.startswith("reserved")}


_lib = None


def lib():
    """The loaded libmpstep.so (raises RuntimeError when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmpstep.so is not built (%s); run __graft_entry__.build()"
                               % _LIB_PATH)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(L):
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    PP = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "mp_status_string": ([i32], ctypes.c_char_p),
        "mp_last_error": ([], ctypes.c_char_p),
        "mp_abi_version": ([], i32),
        "mp_token_weights": ([i32, P, P], i32),
        "mp_state_bytes_per_param": ([i32, i32], ctypes.c_size_t),
        "mp_plan_create": ([i32, P, i32, PP, PP, PP, PP, PP, P, PP], i32),
        "mp_plan_destroy": ([P], i32),
        "mp_plan_info": ([P, P, P, P, P], i32),
        "mp_chunk_layout": ([i32, P, i32, P, P, P, P, P, i64], i32),
        "mp_gradset_create": ([P, PP, PP], i32),
        "mp_gradset_destroy": ([P], i32),
        "mp_state_create": ([ctypes.POINTER(ScalerCfg), PP], i32),
        "mp_state_destroy": ([P], i32),
        "mp_state_read": ([P, P, P], i32),
        "mp_state_scale_ptr": ([P, PP], i32),
        "mp_accumulate": ([P, P, f32, i32, P], i32),
        "mp_unscale_check_norm": ([P, P, P, f32, i32, f32, P], i32),
        "mp_adamw_step": ([P, P, P, f32, i32, ctypes.POINTER(AdamWHparams), P], i32),
        "mp_scaler_update": ([P, P], i32),
        "mp_cast_to_16": ([P, P, i64, i32, P], i32),
        "mp_widen_16": ([P, P, i64, i32, P], i32),
        "mp_state_export": ([P, P, ctypes.c_size_t, P], i32),
        "mp_state_import": ([P, P, ctypes.c_size_t, P], i32),
        "mp_norm_partial": ([P, P, P, f32, i32, P, P], i32),
        "mp_norm_finish": ([P, P, P, f32, P], i32),
        "mp_cast_fp8_blocks": ([P, P, P, i64, i32, P], i32),
        "mp_fp8set_create": ([P, PP, PP, PP], i32),
        "mp_fp8set_destroy": ([P], i32),
        "mp_adamw_step_fp8": ([P, P, P, f32, i32, ctypes.POINTER(AdamWHparams), P, P], i32),
        "mp_gradset_update": ([P, PP, P], i32),
        "mp_update_step": ([P, P, P, f32, i32, f32, ctypes.POINTER(AdamWHparams), P], i32),
        "mp_update_step_noalloc": ([P, P, P, f32, i32, f32, ctypes.POINTER(AdamWHparams), P],
                                   i32),
        "mp_token_weights_dev": ([i32, P, P, P], i32),
        "mp_accumulate_group": ([P, PP, P, i32, i32, i32, P], i32),
        "mp_accumulate_first_counts": ([P, PP, i32, i32, P, P, P], i32),
        "mp_update_step_group": ([P, P, PP, P, i32, i32, i32, f32, ctypes.POINTER(AdamWHparams),
                                  P], i32),
        "mp_unscale_check_norm_group": ([P, P, PP, P, i32, i32, i32, f32, P], i32),
        "mp_adamw_step_group": ([P, P, PP, P, i32, i32, i32, ctypes.POINTER(AdamWHparams), P],
                                i32),
        "mp_norm_partial_group": ([P, P, PP, P, i32, i32, i32, P, P], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def _name(status):
    try:
        return lib().mp_status_string(status).decode()
    except Exception:  # noqa: BLE001 -- naming an error must not raise
        return "status %d" % status


def _check(status):
    if status != MP_OK:
        raise MpError(status, lib().mp_last_error().decode())


def _ptrs(values):
    if values is None:
        return None
    arr = (ctypes.c_void_p * len(values))()
    for i, x in enumerate(values):
        arr[i] = x.data_ptr() if isinstance(x, torch.Tensor) else x
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))


def _addr(x):
    """Device address of a tensor (or an int address); None stays NULL."""
    if x is None:
        return None
    return ctypes.c_void_p(x.data_ptr() if isinstance(x, torch.Tensor) else int(x))


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


# --- the C ABI, one wrapper per entry point -----------------------------------

def mp_status_string(status):
    return lib().mp_status_string(status).decode()


def mp_last_error():
    return lib().mp_last_error().decode()


def mp_abi_version():
    return lib().mp_abi_version()


def mp_token_weights(counts):
    n = (ctypes.c_int64 * len(counts))(*[int(c) for c in counts])
    w = (ctypes.c_float * len(counts))()
    _check(lib().mp_token_weights(len(counts), n, w))
    return list(w)


def mp_token_weights_dev(k, counts, weights_out, stream=None):
    """counts: k int64 on the device; weights_out: k fp32 on the device."""
    _check(lib().mp_token_weights_dev(int(k), _addr(counts), _addr(weights_out),
                                      _stream(stream)))


def mp_state_bytes_per_param(dtype, with_accumulator):
    return lib().mp_state_bytes_per_param(dtype, int(bool(with_accumulator)))


def mp_plan_create(numel, dtype, acc, master, m, v, w16, wd_mult=None):
    n = len(numel)
    ne = (ctypes.c_int64 * n)(*[int(x) for x in numel])
    wd = None if wd_mult is None else (ctypes.c_float * n)(*[float(x) for x in wd_mult])
    out = ctypes.c_void_p()
    _check(lib().mp_plan_create(n, ne, dtype, _ptrs(acc), _ptrs(master), _ptrs(m), _ptrs(v),
                                _ptrs(w16), wd, ctypes.byref(out)))
    return out


def mp_plan_destroy(plan):
    _check(lib().mp_plan_destroy(plan))


def mp_plan_info(plan):
    nt, tot, nc, ce = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(lib().mp_plan_info(plan, ctypes.byref(nt), ctypes.byref(tot), ctypes.byref(nc),
                              ctypes.byref(ce)))
    return {"n_tensors": nt.value, "total_params": tot.value, "n_chunks": nc.value,
            "chunk_elems": ce.value}


def mp_chunk_layout(numel, n_cus):
    """(chunk_elems, [(tensor, start, len), ...]) of the plan mp_plan_create would build."""
    n = len(numel)
    ne = (ctypes.c_int64 * n)(*[int(x) for x in numel])
    ce, nc = ctypes.c_int32(), ctypes.c_int64()
    _check(lib().mp_chunk_layout(n, ne, n_cus, ctypes.byref(ce), ctypes.byref(nc), None, None,
                                 None, 0))
    t = (ctypes.c_int32 * nc.value)()
    s = (ctypes.c_int64 * nc.value)()
    ln = (ctypes.c_int32 * nc.value)()
    _check(lib().mp_chunk_layout(n, ne, n_cus, None, None, t, s, ln, nc.value))
    return ce.value, list(zip(t, s, ln))


def mp_gradset_create(plan, g16):
    out = ctypes.c_void_p()
    _check(lib().mp_gradset_create(plan, _ptrs(g16), ctypes.byref(out)))
    return out


def mp_gradset_update(gradset, g16, stream=None):
    _check(lib().mp_gradset_update(gradset, _ptrs(g16), _stream(stream)))


def mp_gradset_destroy(gradset):
    _check(lib().mp_gradset_destroy(gradset))


def mp_state_create(cfg):
    out = ctypes.c_void_p()
    _check(lib().mp_state_create(ctypes.byref(cfg), ctypes.byref(out)))
    return out


def mp_state_destroy(state):
    _check(lib().mp_state_destroy(state))


def mp_state_read(state, out_ptr, stream=None):
    """Enqueue the copy of the device state into host memory at out_ptr (72 bytes)."""
    _check(lib().mp_state_read(state, ctypes.c_void_p(out_ptr), _stream(stream)))


def mp_state_scale_ptr(state):
    out = ctypes.c_void_p()
    _check(lib().mp_state_scale_ptr(state, ctypes.byref(out)))
    return out.value


def mp_accumulate(plan, gradset, weight, first, stream=None):
    _check(lib().mp_accumulate(plan, gradset, float(weight), int(bool(first)), _stream(stream)))


def _group(sets, weights):
    """(gradset array, weight pointer, on_device) for the *_group entry points: weights is a
    list of floats (host), or a device fp32 tensor or an int device address where len(sets)
    consecutive fp32 weights are read when the kernels run."""
    arr = (ctypes.c_void_p * len(sets))(*[s.value if isinstance(s, ctypes.c_void_p) else s
                                          for s in sets])
    if isinstance(weights, torch.Tensor):
        if not weights.is_cuda or weights.dtype != torch.float32:
            raise TypeError("device weights must be a CUDA float32 tensor")
        return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), _addr(weights), 1
    if isinstance(weights, int):
        return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), _addr(weights), 1
    w = (ctypes.c_float * len(sets))(*[float(x) for x in weights])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), ctypes.cast(w, ctypes.c_void_p), 0


def mp_accumulate_group(plan, sets, weights, first, stream=None):
    """Accumulate len(sets) resident micro-batches in one pass (see mp_accumulate_group)."""
    arr, w, dev = _group(sets, weights)
    _check(lib().mp_accumulate_group(plan, arr, w, len(sets), dev, int(bool(first)),
                                     _stream(stream)))


def mp_accumulate_first_counts(plan, sets, k, counts, weights_out, stream=None):
    """Token weights from device counts computed inside the first accumulation of sets (see
    the header); weights_out receives all k weights for the later passes."""
    arr = (ctypes.c_void_p * len(sets))(*[x.value if isinstance(x, ctypes.c_void_p) else x
                                          for x in sets])
    _check(lib().mp_accumulate_first_counts(plan, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)),
                                            len(sets), int(k), _addr(counts), _addr(weights_out),
                                            _stream(stream)))


def mp_unscale_check_norm(plan, state, last, w_last, last_is_first, max_norm, stream=None):
    _check(lib().mp_unscale_check_norm(plan, state, last, float(w_last), int(bool(last_is_first)),
                                       float(max_norm), _stream(stream)))


def mp_adamw_step(plan, state, last, w_last, last_is_first, hp, stream=None):
    _check(lib().mp_adamw_step(plan, state, last, float(w_last), int(bool(last_is_first)),
                               ctypes.byref(hp), _stream(stream)))


def mp_update_step(plan, state, last, w_last, last_is_first, max_norm, hp, stream=None):
    _check(lib().mp_update_step(plan, state, last, float(w_last), int(bool(last_is_first)),
                                float(max_norm), ctypes.byref(hp), _stream(stream)))


def mp_update_step_noalloc(plan, state, last, w_last, last_is_first, max_norm, hp, stream=None):
    """mp_update_step with the norm's scratch in the library's static device array."""
    _check(lib().mp_update_step_noalloc(plan, state, last, float(w_last),
                                        int(bool(last_is_first)), float(max_norm),
                                        ctypes.byref(hp), _stream(stream)))


def mp_unscale_check_norm_group(plan, state, sets, weights, last_is_first, max_norm,
                                stream=None):
    arr, w, dev = _group(sets, weights)
    _check(lib().mp_unscale_check_norm_group(plan, state, arr, w, len(sets), dev,
                                             int(bool(last_is_first)), float(max_norm),
                                             _stream(stream)))


def mp_norm_partial_group(plan, state, sets, weights, last_is_first, partial_out, stream=None):
    arr, w, dev = _group(sets, weights)
    _check(lib().mp_norm_partial_group(plan, state, arr, w, len(sets), dev,
                                       int(bool(last_is_first)), _addr(partial_out),
                                       _stream(stream)))


def mp_adamw_step_group(plan, state, sets, weights, last_is_first, hp, stream=None):
    arr, w, dev = _group(sets, weights)
    _check(lib().mp_adamw_step_group(plan, state, arr, w, len(sets), dev,
                                     int(bool(last_is_first)), ctypes.byref(hp), _stream(stream)))


def mp_update_step_group(plan, state, sets, weights, last_is_first, max_norm, hp, stream=None):
    """mp_update_step with len(sets) resident micro-batches folded in (see the header)."""
    arr, w, dev = _group(sets, weights)
    _check(lib().mp_update_step_group(plan, state, arr, w, len(sets), dev,
                                      int(bool(last_is_first)), float(max_norm),
                                      ctypes.byref(hp), _stream(stream)))


def mp_scaler_update(state, stream=None):
    _check(lib().mp_scaler_update(state, _stream(stream)))


def mp_cast_to_16(src, dst, n, dtype, stream=None):
    _check(lib().mp_cast_to_16(ctypes.c_void_p(src), ctypes.c_void_p(dst), int(n), dtype,
                               _stream(stream)))


def mp_widen_16(src, dst, n, dtype, stream=None):
    _check(lib().mp_widen_16(ctypes.c_void_p(src), ctypes.c_void_p(dst), int(n), dtype,
                             _stream(stream)))


def mp_state_export(state, blob_ptr, blob_bytes=MP_STATE_BLOB_BYTES, stream=None):
    _check(lib().mp_state_export(state, ctypes.c_void_p(blob_ptr), blob_bytes, _stream(stream)))


def mp_state_import(state, blob_ptr, blob_bytes=MP_STATE_BLOB_BYTES, stream=None):
    _check(lib().mp_state_import(state, ctypes.c_void_p(blob_ptr), blob_bytes, _stream(stream)))


def mp_norm_partial(plan, state, last, w_last, last_is_first, partial_out, stream=None):
    _check(lib().mp_norm_partial(plan, state, last, float(w_last), int(bool(last_is_first)),
                                 ctypes.c_void_p(partial_out), _stream(stream)))


def mp_norm_finish(plan, state, sumsq, max_norm, stream=None):
    _check(lib().mp_norm_finish(plan, state, ctypes.c_void_p(sumsq), float(max_norm),
                                _stream(stream)))


def mp_cast_fp8_blocks(src, codes, scales, n, block=16, stream=None):
    _check(lib().mp_cast_fp8_blocks(ctypes.c_void_p(src), ctypes.c_void_p(codes),
                                    ctypes.c_void_p(scales), int(n), int(block), _stream(stream)))


def mp_fp8set_create(plan, codes, scales):
    """codes[i], scales[i]: tensors / device addresses, or None for a tensor that is not cast."""
    out = ctypes.c_void_p()
    _check(lib().mp_fp8set_create(plan, _ptrs(codes), _ptrs(scales), ctypes.byref(out)))
    return out


def mp_fp8set_destroy(fp8set):
    _check(lib().mp_fp8set_destroy(fp8set))


def mp_adamw_step_fp8(plan, state, last, w_last, last_is_first, hp, fp8set, stream=None):
    _check(lib().mp_adamw_step_fp8(plan, state, last, float(w_last), int(bool(last_is_first)),
                                   ctypes.byref(hp), fp8set, _stream(stream)))


# --- convenience ---------------------------------------------------------------

def scaler_cfg(init_scale=2.0 ** 16, growth=2.0, backoff=0.5, min_scale=1.0, max_scale=2.0 ** 64,
               interval=2000, enabled=True):
    return ScalerCfg(init_scale, growth, backoff, min_scale, max_scale, interval, int(bool(enabled)))


def adamw_hparams(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1):
    return AdamWHparams(lr, beta1, beta2, eps, weight_decay)


def save_state(state, stream=None):
    """The state blob as bytes (enqueues the copy, then waits for the stream)."""
    buf = torch.empty(MP_STATE_BLOB_BYTES, dtype=torch.uint8, pin_memory=True)
    s = stream if stream is not None else torch.cuda.current_stream()
    mp_state_export(state, buf.data_ptr(), MP_STATE_BLOB_BYTES, s)
    s.synchronize()
    return bytes(buf.numpy())


def load_state(state, blob, stream=None):
    buf = ctypes.create_string_buffer(bytes(blob), len(blob))
    mp_state_import(state, ctypes.addressof(buf), len(blob), stream)


def read_stats(state, stream=None):
    """Read the device state (enqueues the copy, then waits for the stream)."""
    buf = torch.empty(ctypes.sizeof(Stats), dtype=torch.uint8, pin_memory=True)
    s = stream if stream is not None else torch.cuda.current_stream()
    mp_state_read(state, buf.data_ptr(), s)
    s.synchronize()
    return Stats.from_buffer_copy(bytes(buf.numpy())).as_dict()


# Tensor starts in the flat layout: a multiple of 64 elements (256 B of fp32, 128 B of a 16-bit
# format).  The library needs 16 bytes; whole cache lines keep the AdamW pass from writing
# partial lines at every tensor edge, which cost it 10% on a list of 4096 ragged tensors.
FLAT_ALIGN_ELEMS = 64


def _align_elems(n):
    return (n + FLAT_ALIGN_ELEMS - 1) // FLAT_ALIGN_ELEMS * FLAT_ALIGN_ELEMS


class ModelState:
    """Device buffers of one model (torch allocations) and the plan over them.

    For each tensor: fp32 master, m, v, the 16-bit weight, and (with_acc) the
    fp32 accumulation buffer.  ``layout="tensor"`` allocates every buffer of
    every tensor separately; ``layout="flat"`` allocates one contiguous buffer
    per kind (Megatron-style flattened buffers) and hands the plan per-tensor
    views into it, each starting on a multiple of ``FLAT_ALIGN_ELEMS`` (64)
    elements.  ``g16`` gradient buffers are the caller's;
    ``grad_buffers`` makes them in the same layout.
    """

    def __init__(self, numels, dtype, with_acc=True, wd_mult=None, device="cuda",
                 layout="tensor"):
        self.numels = [int(n) for n in numels]
        self.dtype = dtype
        self.layout = layout
        self.device = device
        self.t16 = torch.bfloat16 if dtype == MP_BF16 else torch.float16
        self.master = self._alloc(torch.float32)
        self.m = self._alloc(torch.float32, zero=True)
        self.v = self._alloc(torch.float32, zero=True)
        self.w16 = self._alloc(self.t16, zero=True)
        self.acc = self._alloc(torch.float32, zero=True) if with_acc else None
        self.plan = mp_plan_create(self.numels, dtype, self.acc, self.master, self.m, self.v,
                                   self.w16, wd_mult)

    def _alloc(self, dt, zero=False):
        make = torch.zeros if zero else torch.empty
        if self.layout == "tensor":
            return [make(n, dtype=dt, device=self.device) for n in self.numels]
        assert self.layout == "flat", self.layout
        offs, total = [], 0
        for n in self.numels:
            offs.append(total)
            total += _align_elems(n)
        flat = make(total, dtype=dt, device=self.device)
        return [flat[o:o + n] for o, n in zip(offs, self.numels)]

    def grad_buffers(self):
        """One micro-batch's 16-bit gradient buffers, in this model's layout."""
        return self._alloc(self.t16)

    def gradset(self, g16):
        return mp_gradset_create(self.plan, g16)

    def close(self):
        if self.plan:
            mp_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass
