"""CPU oracle of the error-bounded float32 codec -- TEST INFRASTRUCTURE ONLY.

This package wraps ``eblc_oracle.cpp`` (plain single-threaded C++, fp32 without FMA
contraction) through ctypes.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import it; the product library never does, and the two
share no code.  See ``eblc_oracle.h`` for what each function computes and which passage
of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eblc_oracle.cpp")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "liboracle.so")

OK = 0
CAPACITY = 3
CORRUPT = 4


def build() -> str:
    """Compile the oracle with g++ (-O2, no FMA contraction, no fast-math)."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    tmp = _LIB + ".tmp"
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        u64, i32, u32, f64 = ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32, ctypes.c_double
        L.oracle_resolve_bound.argtypes = [P, u64, i32, f64, P, P, P]
        L.oracle_resolve_bound.restype = i32
        L.oracle_quantize_one.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_float, i32, P]
        L.oracle_quantize_one.restype = i32
        L.oracle_codes.argtypes = [P, u64, ctypes.c_float, ctypes.c_float, ctypes.c_float, i32,
                                   u32, P, P, P, P, P]
        L.oracle_codes.restype = None
        L.oracle_pack.argtypes = [P, u64, P, P]
        L.oracle_pack.restype = u64
        L.oracle_unpack_one.argtypes = [P, u32, u32]
        L.oracle_unpack_one.restype = u32
        L.oracle_stream_bytes.argtypes = [u64, u64, u64]
        L.oracle_stream_bytes.restype = u64
        L.oracle_raw_bytes.argtypes = [u64]
        L.oracle_raw_bytes.restype = u64
        L.oracle_compress.argtypes = [P, i32, P, i32, f64, u32, i32, u64, P, u64, P]
        L.oracle_compress.restype = u64
        L.oracle_decompress.argtypes = [P, u64, P, u64]
        L.oracle_decompress.restype = i32
        L.oracle_stream_elements.argtypes = [P, u64]
        L.oracle_stream_elements.restype = u64
        L.oracle_block_means.argtypes = [P, u64, u32, P]
        L.oracle_block_means.restype = None
        L.oracle_stream_bytes_centered.argtypes = [u64, u32, u64, u64]
        L.oracle_stream_bytes_centered.restype = u64
        L.oracle_compress_ex.argtypes = [P, i32, P, i32, f64, u32, i32, u64, i32, P, u64, P]
        L.oracle_compress_ex.restype = u64
        L.oracle_bitshuffle.argtypes = [P, u32, P]
        L.oracle_bitshuffle.restype = None
        L.oracle_unbitshuffle.argtypes = [P, u32, P]
        L.oracle_unbitshuffle.restype = None
        L.oracle_rze.argtypes = [P, u32, P]
        L.oracle_rze.restype = u32
        L.oracle_unrze.argtypes = [P, u32, u32, P]
        L.oracle_unrze.restype = i32
        L.oracle_chunk_stream_bytes.argtypes = [u64, u32, u64, u64]
        L.oracle_chunk_stream_bytes.restype = u64
        L.oracle_compress_chunked.argtypes = [P, i32, P, i32, f64, u32, i32, u64, P, u64, P]
        L.oracle_compress_chunked.restype = u64
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def resolve_bound(x: np.ndarray, rel: bool, eps: float):
    """Returns (valid, eb_f, s, r) as numpy float32 scalars."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(3, dtype=np.float32)
    o = out.ctypes.data
    v = lib().oracle_resolve_bound(_ptr(x), x.size, int(rel), float(eps),
                                   ctypes.c_void_p(o), ctypes.c_void_p(o + 4),
                                   ctypes.c_void_p(o + 8))
    return bool(v), out[0], out[1], out[2]


def quantize_one(x: float, eb_f, s, r, T: int):
    """Returns the code, or None if the value escapes."""
    q = np.zeros(1, dtype=np.int32)
    e = lib().oracle_quantize_one(ctypes.c_float(np.float32(x)), ctypes.c_float(eb_f),
                                  ctypes.c_float(s), ctypes.c_float(r), T, _ptr(q))
    return None if e else int(q[0])


def codes(x: np.ndarray, eb_f, s, r, T: int, B: int):
    """Steps 2-5: returns dict of q, esc, d, z, widths."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.size
    q = np.zeros(n, np.int32)
    esc = np.zeros(n, np.uint8)
    d = np.zeros(n, np.int32)
    z = np.zeros(n, np.uint32)
    w = np.zeros((n + 31) // 32, np.uint8)
    lib().oracle_codes(_ptr(x), n, ctypes.c_float(eb_f), ctypes.c_float(s), ctypes.c_float(r),
                       T, B, _ptr(q), _ptr(esc), _ptr(d), _ptr(z), _ptr(w))
    return {"q": q, "esc": esc, "d": d, "z": z, "widths": w}


def pack(z: np.ndarray, widths: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.uint32)
    widths = np.ascontiguousarray(widths, dtype=np.uint8)
    words = np.zeros(int(widths.astype(np.uint64).sum()) + 1, np.uint32)
    nw = lib().oracle_pack(_ptr(z), z.size, _ptr(widths), _ptr(words))
    return words[:nw]


def stream_bytes(n: int, sum_widths: int, m: int) -> int:
    return int(lib().oracle_stream_bytes(n, sum_widths, m))


def raw_bytes(n: int) -> int:
    return int(lib().oracle_raw_bytes(n))


def compress(x: np.ndarray, dims, rel: bool, eps: float, B: int = 256, T: int = 30,
             side_max: int | None = None, center: bool = False) -> np.ndarray:
    """Whole compressor; returns the stream as a uint8 array.  center: Lorenzo centering."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    dims = [int(v) for v in dims]
    n = int(np.prod(dims))
    assert n == x.size
    if side_max is None:
        side_max = min(n, 1 << 23)
    d = np.asarray(dims, dtype=np.uint64)
    cap = raw_bytes(n)
    out = np.zeros(cap, np.uint8)
    req = np.zeros(1, np.uint64)
    tot = lib().oracle_compress_ex(_ptr(x), len(dims), _ptr(d), int(rel), float(eps), B, T,
                                   side_max, int(center), _ptr(out), cap, _ptr(req))
    assert tot > 0, "oracle stream larger than the raw bound"
    return out[:tot].copy()


def compress_chunked(x: np.ndarray, dims, rel: bool, eps: float, chunk_values: int = 2048, T: int = 30,
                     side_max: int | None = None) -> np.ndarray:
    """Whole compressor with the chunk-cooperative coder (chunk_values = 1024, 2048 or 4096)."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    dims = [int(v) for v in dims]
    n = int(np.prod(dims))
    assert n == x.size
    if side_max is None:
        side_max = min(n, 1 << 23)
    d = np.asarray(dims, dtype=np.uint64)
    cap = raw_bytes(n)
    out = np.zeros(cap, np.uint8)
    req = np.zeros(1, np.uint64)
    tot = lib().oracle_compress_chunked(_ptr(x), len(dims), _ptr(d), int(rel), float(eps), chunk_values, T,
                                        side_max, _ptr(out), cap, _ptr(req))
    assert tot > 0, "oracle stream larger than the raw bound"
    return out[:tot].copy()


def block_means(q: np.ndarray, B: int) -> np.ndarray:
    """Lorenzo centering: each block's mean code, rounded half up."""
    q = np.ascontiguousarray(q, dtype=np.int32)
    out = np.zeros((q.size + B - 1) // B, np.int32)
    lib().oracle_block_means(_ptr(q), q.size, B, _ptr(out))
    return out


def stream_bytes_centered(n: int, B: int, sum_widths: int, m: int) -> int:
    return int(lib().oracle_stream_bytes_centered(n, B, sum_widths, m))


def bitshuffle(z: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.uint32)
    w = np.zeros(z.size, np.uint32)
    lib().oracle_bitshuffle(_ptr(z), z.size, _ptr(w))
    return w


def unbitshuffle(words: np.ndarray) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint32)
    z = np.zeros(words.size, np.uint32)
    lib().oracle_unbitshuffle(_ptr(words), words.size, _ptr(z))
    return z


def rze(words: np.ndarray) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint32)
    out = np.zeros(words.size + words.size // 32, np.uint32)
    k = lib().oracle_rze(_ptr(words), words.size, _ptr(out))
    return out[:k].copy()


def unrze(data: np.ndarray, W: int):
    """Returns the W words, or None for an inconsistent input."""
    data = np.ascontiguousarray(data, dtype=np.uint32)
    words = np.zeros(W, np.uint32)
    st = lib().oracle_unrze(_ptr(data) if data.size else None, data.size, W, _ptr(words))
    return None if st != 0 else words


def chunk_stream_bytes(n: int, V: int, sum_words: int, m: int) -> int:
    return int(lib().oracle_chunk_stream_bytes(n, V, sum_words, m))


def decompress(stream: np.ndarray, n: int | None = None):
    """Returns (status, x') with x' float32 of the stream's element count."""
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    if n is None:
        n = int(lib().oracle_stream_elements(_ptr(stream), stream.size))
    out = np.zeros(max(n, 1), np.float32)
    st = lib().oracle_decompress(_ptr(stream), stream.size, _ptr(out), n)
    return int(st), out[:n]


def stream_elements(stream: np.ndarray) -> int:
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    return int(lib().oracle_stream_elements(_ptr(stream), stream.size))
