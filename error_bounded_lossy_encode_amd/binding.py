"""ctypes binding of libeblc.so (C ABI in include/eblc.h), same function names.

Argument marshalling only: every step of the codec runs in the library's HIP kernels.  Device
buffers are torch tensors on the plan's device; streams are torch streams (or None for the
current stream).  Loading fails loudly when the library has not been built -- there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libeblc.so")

EBLC_OK = 0
EBLC_UNSUPPORTED = 1
EBLC_INVALID_ARGUMENT = 2
EBLC_CAPACITY = 3
EBLC_CORRUPT_STREAM = 4
EBLC_DEVICE_ERROR = 5
EBLC_OUT_OF_MEMORY = 6
EBLC_TOO_LARGE = 7

EBLC_EXECUTION_HOST = 0
EBLC_EXECUTION_CUDA = 1
EBLC_EXECUTION_HIP = 2
EBLC_FLOAT32 = 0
HEADER_BYTES = 128


class eblc_execution_t(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("device", ctypes.c_int), ("threads", ctypes.c_int)]


class eblc_result_t(ctypes.Structure):
    _fields_ = [("compressed_bytes", ctypes.c_uint64), ("status", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


class eblc_limits_t(ctypes.Structure):
    _fields_ = [("max_compressed_bytes", ctypes.c_size_t), ("payload_alignment", ctypes.c_size_t),
                ("sidecar_bytes", ctypes.c_size_t), ("sidecar_alignment", ctypes.c_size_t)]


EXPORTS = ["eblc_abi_version", "eblc_plan_create", "eblc_plan_limits", "eblc_max_compressed_bytes",
           "eblc_payload_alignment", "eblc_compress", "eblc_compress_async", "eblc_compress_noalloc",
           "eblc_compress_batch",
           "eblc_decompress", "eblc_decompress_batch", "eblc_plan_status", "eblc_plan_destroy", "eblc_status_string",
           "eblc_plan_set_profiling", "eblc_plan_kernel_times"]

_lib = None


def lib():
    """Load libeblc.so; raises if it is missing (build it with __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libeblc.so not built ({LIB_PATH}); run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.eblc_abi_version.argtypes = []
    L.eblc_abi_version.restype = I
    L.eblc_plan_create.argtypes = [ctypes.POINTER(eblc_execution_t), I, I, P, P, ctypes.c_char_p,
                                   ctypes.POINTER(P)]
    L.eblc_plan_create.restype = I
    L.eblc_plan_limits.argtypes = [P, ctypes.POINTER(eblc_limits_t)]
    L.eblc_plan_limits.restype = I
    L.eblc_max_compressed_bytes.argtypes = [P]
    L.eblc_max_compressed_bytes.restype = SZ
    L.eblc_payload_alignment.argtypes = [P]
    L.eblc_payload_alignment.restype = SZ
    L.eblc_compress.argtypes = [P, P, P, SZ, ctypes.POINTER(SZ), P, P]
    L.eblc_compress.restype = I
    L.eblc_compress_async.argtypes = [P, P, P, SZ, P, P]
    L.eblc_compress_async.restype = I
    L.eblc_compress_noalloc.argtypes = [ctypes.POINTER(eblc_execution_t), I, P, P, ctypes.c_char_p, P, P, SZ, P, P]
    L.eblc_compress_noalloc.restype = I
    L.eblc_compress_batch.argtypes = [P, I, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(SZ), P, P]
    L.eblc_compress_batch.restype = I
    L.eblc_decompress.argtypes = [P, P, SZ, P, P, P]
    L.eblc_decompress.restype = I
    L.eblc_decompress_batch.argtypes = [P, I, ctypes.POINTER(P), ctypes.POINTER(SZ), ctypes.POINTER(P), P]
    L.eblc_decompress_batch.restype = I
    L.eblc_plan_status.argtypes = [P, P]
    L.eblc_plan_status.restype = I
    L.eblc_plan_destroy.argtypes = [P]
    L.eblc_plan_destroy.restype = None
    L.eblc_status_string.argtypes = [I]
    L.eblc_status_string.restype = ctypes.c_char_p
    L.eblc_plan_set_profiling.argtypes = [P, I, ctypes.c_char_p, I]
    L.eblc_plan_set_profiling.restype = I
    L.eblc_plan_kernel_times.argtypes = [P, ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(ctypes.c_float), ctypes.POINTER(I), I]
    L.eblc_plan_kernel_times.restype = I
    _lib = L
    return L


def _stream_handle(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def eblc_abi_version() -> int:
    return int(lib().eblc_abi_version())


def eblc_status_string(status: int) -> str:
    return lib().eblc_status_string(int(status)).decode()


def eblc_plan_create(dims, options: str | None = None, device: int = 0, strides=None,
                     kind: int = EBLC_EXECUTION_HIP, dtype: int = EBLC_FLOAT32):
    """Returns (status, plan handle or None).  dims slowest to fastest."""
    dims = [int(d) for d in dims]
    d = (ctypes.c_int64 * max(1, len(dims)))(*dims)
    s = None
    if strides is not None:
        s = (ctypes.c_int64 * len(strides))(*[int(v) for v in strides])
    ex = eblc_execution_t(kind, device, 0)
    plan = ctypes.c_void_p()
    st = lib().eblc_plan_create(ctypes.byref(ex), dtype, len(dims), d, s,
                                None if options is None else options.encode(), ctypes.byref(plan))
    return st, (plan if st == EBLC_OK else None)


def eblc_plan_limits(plan):
    lim = eblc_limits_t()
    st = lib().eblc_plan_limits(plan, ctypes.byref(lim))
    return st, {f: int(getattr(lim, f)) for f, _ in eblc_limits_t._fields_}


def eblc_max_compressed_bytes(plan) -> int:
    return int(lib().eblc_max_compressed_bytes(plan))


def eblc_payload_alignment(plan) -> int:
    return int(lib().eblc_payload_alignment(plan))


def eblc_compress(plan, x, out, out_capacity: int | None = None, stream=None):
    """x: float32 device tensor; out: uint8 device tensor.  Returns (status, compressed_bytes)."""
    cap = out.numel() * out.element_size() if out_capacity is None else int(out_capacity)
    nbytes = ctypes.c_size_t(0)
    st = lib().eblc_compress(plan, _ptr(x), _ptr(out), cap, ctypes.byref(nbytes), None,
                             _stream_handle(stream))
    return st, int(nbytes.value)


def eblc_compress_async(plan, x, out, result, out_capacity: int | None = None, stream=None) -> int:
    """x: float32 device tensor; out: uint8 device tensor; result: a device tensor of >= 16 bytes
    (or a pinned host one) that receives the eblc_result_t record.  Returns the status."""
    cap = out.numel() * out.element_size() if out_capacity is None else int(out_capacity)
    return int(lib().eblc_compress_async(plan, _ptr(x), _ptr(out), cap, _ptr(result),
                                         _stream_handle(stream)))


def eblc_compress_noalloc(dims, options, x, out, result, out_capacity: int | None = None, device: int = 0,
                          strides=None, stream=None) -> int:
    """Plan-less compress into the library's static scratch: x float32 device tensor, out uint8
    device tensor, result a device (or pinned host) tensor of >= 16 bytes receiving the
    eblc_result_t record.  Returns the status."""
    dims = [int(d) for d in dims]
    d = (ctypes.c_int64 * max(1, len(dims)))(*dims)
    s = None if strides is None else (ctypes.c_int64 * len(strides))(*[int(v) for v in strides])
    ex = eblc_execution_t(EBLC_EXECUTION_HIP, device, 0)
    cap = out.numel() * out.element_size() if out_capacity is None else int(out_capacity)
    return int(lib().eblc_compress_noalloc(ctypes.byref(ex), len(dims), d, s,
                                           None if options is None else options.encode(), _ptr(x), _ptr(out),
                                           cap, _ptr(result), _stream_handle(stream)))


def eblc_compress_batch(plan, xs, outs, results, capacities=None, stream=None) -> int:
    """Enqueue len(xs) compressions back to back; results: one device (or pinned host) tensor
    holding len(xs) eblc_result_t records (16 bytes each).  Returns the status."""
    k = len(xs)
    ins = (ctypes.c_void_p * max(k, 1))(*[t.data_ptr() for t in xs])
    os_ = (ctypes.c_void_p * max(k, 1))(*[t.data_ptr() for t in outs])
    caps = [t.numel() * t.element_size() for t in outs] if capacities is None else capacities
    cs = (ctypes.c_size_t * max(k, 1))(*[int(c) for c in caps])
    return int(lib().eblc_compress_batch(plan, k, ins, os_, cs, _ptr(results), _stream_handle(stream)))


def eblc_decompress_batch(plan, streams, ys, sizes=None, stream=None) -> int:
    """Enqueue len(streams) decompressions (uint8 device tensors -> float32 device tensors);
    sizes: readable bytes of each stream (default: its tensor's size).  Returns the status."""
    k = len(streams)
    ins = (ctypes.c_void_p * max(k, 1))(*[t.data_ptr() for t in streams])
    outs = (ctypes.c_void_p * max(k, 1))(*[t.data_ptr() for t in ys])
    szs = [t.numel() * t.element_size() for t in streams] if sizes is None else sizes
    cs = (ctypes.c_size_t * max(k, 1))(*[int(c) for c in szs])
    return int(lib().eblc_decompress_batch(plan, k, ins, cs, outs, _stream_handle(stream)))


def result_records(results) -> list:
    """[(compressed_bytes, status)] from a tensor of eblc_result_t records (copied to host)."""
    import numpy as np
    raw = results.cpu().numpy().view(np.uint8).reshape(-1)
    recs = raw[: raw.size // 16 * 16].view(np.uint64).reshape(-1, 2)
    return [(int(r[0]), int(r[1] & 0xFFFFFFFF)) for r in recs]


def eblc_decompress(plan, stream_buf, compressed_bytes: int, out, stream=None) -> int:
    """stream_buf: uint8 device tensor holding the stream; out: float32 device tensor."""
    return int(lib().eblc_decompress(plan, _ptr(stream_buf), int(compressed_bytes), None, _ptr(out),
                                     _stream_handle(stream)))


def eblc_plan_status(plan, stream=None) -> int:
    return int(lib().eblc_plan_status(plan, _stream_handle(stream)))


def eblc_plan_destroy(plan) -> None:
    if plan is not None:
        lib().eblc_plan_destroy(plan)


def eblc_plan_set_profiling(plan, max_launches: int, kernels: str | None = None, every: int = 1) -> int:
    """Record an event pair around each of the plan's next max_launches launches (0: off) of
    the kernels named in the comma-separated `kernels` (None: every kernel), in every
    every-th compress and decompress launch sequence."""
    return int(lib().eblc_plan_set_profiling(plan, int(max_launches),
                                             None if kernels is None else kernels.encode(), int(every)))


def eblc_plan_kernel_times(plan, max_kernels: int = 16):
    """[(kernel name, mean milliseconds, launches)] over the launches recorded since the last
    read, in order of first launch; clears the records."""
    names = (ctypes.c_char_p * max_kernels)()
    ms = (ctypes.c_float * max_kernels)()
    cnt = (ctypes.c_int * max_kernels)()
    k = lib().eblc_plan_kernel_times(plan, names, ms, cnt, max_kernels)
    if k < 0:
        raise RuntimeError("kernel times unavailable (profiling off or device error)")
    return [(names[i].decode(), float(ms[i]), int(cnt[i])) for i in range(min(k, max_kernels))]


class Plan:
    """Owning wrapper: a plan plus its limits; destroys the plan when closed."""

    def __init__(self, dims, options: str | None = None, device: int = 0, strides=None):
        st, p = eblc_plan_create(dims, options, device, strides=strides)
        if st != EBLC_OK:
            raise ValueError(f"eblc_plan_create: {eblc_status_string(st)}")
        self.handle = p
        self.dims = [int(d) for d in dims]
        self.n = 1
        for d in self.dims:
            self.n *= d
        self.device = device
        self.max_bytes = eblc_max_compressed_bytes(p)

    def close(self):
        if self.handle is not None:
            eblc_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
