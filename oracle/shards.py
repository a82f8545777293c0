"""Sharded runs of the unchanged oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests and the benchmark's CPU-baseline leg use this module; it shares nothing with the
product library.

Every coded unit of the stream -- a Lorenzo block with its mean, a 32-value segment and its
width, a chunk of the chunk coder, an outlier -- lies inside one piece of a field cut along its
flattened index at multiples of the block (or chunk) length.  So the field can be coded piece by
piece with the oracle, all pieces under the bound resolved once on the whole field (passed in
absolute mode: an fp32 bound given as eps is taken as it is), and the pieces' sections joined
in order: widths (or chunk word counts), block means, payload words, outlier indices shifted by
the piece's start, outlier values; the offset table is then taken again from the joined sizes.  The joined stream must equal the whole-field stream byte for
byte, and the pieces can be coded on as many threads as there are pieces (ctypes releases the
interpreter lock during each oracle call).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

HEADER = 128
GROUP_VALUES = 8192  # values per entry of the stream's offset table


def _align16(v: int) -> int:
    return (v + 15) // 16 * 16


def piece_bounds(n: int, pieces: int, align: int):
    """[start, end) of up to `pieces` pieces of n values, every start a multiple of align."""
    units = (n + align - 1) // align
    pieces = max(1, min(pieces, units))
    cuts = [(units * k // pieces) * align for k in range(pieces)] + [n]
    return [(cuts[k], min(cuts[k + 1], n)) for k in range(pieces) if cuts[k] < min(cuts[k + 1], n)]


def _header(s: np.ndarray) -> dict:
    u32 = s[:HEADER].view(np.uint32)
    u64 = s[:HEADER].view(np.uint64)
    return {"mode": int(s[8]), "n": int(u64[6]), "flags": int(u32[17]), "m": int(u64[9]),
            "pb": int(u64[10]), "po": int(u64[12]), "oi": int(u64[13]), "ov": int(u64[14]),
            "B": int(u32[3])}


def code_pieces(x: np.ndarray, rel: bool, eps: float, B: int, T: int, center: bool, V: int | None,
                pieces: int, threads: int):
    """The field's bound, its pieces and each piece's oracle stream (coded on `threads` threads).
    Returns (valid, eb_f, bounds, streams)."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    valid, eb_f, _, _ = oracle.resolve_bound(x, rel, eps)
    bounds = piece_bounds(x.size, pieces, V if V else max(B, 32))

    def one(ab):
        a, b = ab
        xs = x[a:b]
        if V:
            return oracle.compress_chunked(xs, [b - a], False, float(eb_f), V, T, b - a)
        return oracle.compress(xs, [b - a], False, float(eb_f), B, T, b - a, center=center)

    if not valid:
        return False, eb_f, bounds, []
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        streams = list(ex.map(one, bounds))
    return True, eb_f, bounds, streams


def decode_pieces(streams, threads: int):
    """Each piece's stream decoded by the oracle on `threads` threads; the concatenated values."""
    def one(s):
        st, y = oracle.decompress(s)
        assert st == oracle.OK
        return y

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return np.concatenate(list(ex.map(one, streams)))


def join(x: np.ndarray, dims, T: int, B: int, side_max: int, center: bool, V: int | None, bounds,
         streams) -> np.ndarray | None:
    """The whole-field stream from the pieces' streams, with the oracle's layout and RAW rule;
    None when a piece fell back to a raw copy (its sections are then not available)."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    n = x.size
    hs = [_header(s) for s in streams]
    if any(h["mode"] == 1 for h in hs):
        return None
    rank = len(dims)
    h0 = streams[0][:HEADER].copy()
    u32_0 = h0.view(np.uint32)
    eb_f, s_, r_ = u32_0[14], u32_0[15], u32_0[16]
    sizes, means, pay, oidx, oval = [], [], [], [], []
    for (a, b), s, h in zip(bounds, streams, hs):
        ni = b - a
        if V:
            nc = (ni + V - 1) // V
            sizes.append(s[HEADER:HEADER + 4 * nc])
        else:
            nseg = (ni + 31) // 32
            sizes.append(s[HEADER:HEADER + nseg])
            if center:
                nb = (ni + B - 1) // B
                pm = HEADER + _align16(nseg) + _align16(4 * ((ni + GROUP_VALUES - 1) // GROUP_VALUES - 1))
                means.append(s[pm:pm + 4 * nb])
        pay.append(s[h["po"]:h["po"] + h["pb"]])
        oidx.append(s[h["oi"]:h["oi"] + 4 * h["m"]].view(np.uint32) + np.uint32(a))
        oval.append(s[h["ov"]:h["ov"] + 4 * h["m"]])
    sizes = np.concatenate(sizes)
    pay = np.concatenate(pay)
    m = int(sum(h["m"] for h in hs))
    sum_words = pay.size // 4
    if V:
        coded = oracle.chunk_stream_bytes(n, V, sum_words, m)
    elif center:
        coded = oracle.stream_bytes_centered(n, B, sum_words, m)
    else:
        coded = oracle.stream_bytes(n, sum_words, m)
    raw_total = oracle.raw_bytes(n)
    out_dims = [int(d) for d in dims] + [0] * (4 - rank)
    hdr = np.zeros(HEADER, np.uint8)
    hu32, hu64 = hdr.view(np.uint32), hdr.view(np.uint64)
    hu32[0] = u32_0[0]
    hu32[1] = u32_0[1]
    hu32[3] = V if V else B
    for k in range(4):
        hu64[2 + k] = out_dims[k]
    hu64[6] = n
    hu32[14], hu32[15], hu32[16] = eb_f, s_, r_
    hu64[11] = HEADER
    if m > side_max or coded > raw_total:
        hdr[8], hdr[9], hdr[11] = 1, rank, T
        hdr[10] = int(V).bit_length() - 1 if V else 5
        hu64[9], hu64[10], hu64[12] = 0, 4 * n, HEADER
        hu64[13] = hu64[14] = hu64[15] = raw_total
        out = np.zeros(raw_total, np.uint8)
        out[:HEADER] = hdr
        out[HEADER:HEADER + 4 * n] = x.view(np.uint8)
        return out
    hdr[8] = 2 if V else 0
    hdr[9], hdr[11] = rank, T
    hdr[10] = int(V).bit_length() - 1 if V else 5
    size_sec = _align16(sizes.size)
    # the offset table after the size section: payload words before each group of GROUP_VALUES
    # values after the first
    unit_words = sizes.view(np.uint32).astype(np.int64) if V else sizes.astype(np.int64)
    per_group = GROUP_VALUES // (V if V else 32)
    starts = np.arange(per_group, unit_words.size, per_group)
    table = np.concatenate([[0], np.cumsum(unit_words)])[starts].astype(np.uint32)
    tab = HEADER + size_sec
    msec = _align16(4 * ((n + B - 1) // B)) if (center and not V) else 0
    moff = tab + _align16(4 * table.size)
    po = moff + msec
    oi = po + _align16(pay.size)
    ov = oi + _align16(4 * m)
    total = ov + _align16(4 * m)
    hu32[17] = 1 if (center and not V) else 0
    hu64[9], hu64[10], hu64[12], hu64[13], hu64[14], hu64[15] = m, pay.size, po, oi, ov, total
    out = np.zeros(total, np.uint8)
    out[:HEADER] = hdr
    out[HEADER:HEADER + sizes.size] = sizes
    if msec:
        mm = np.concatenate(means)
        out[moff:moff + mm.size] = mm
    out[po:po + pay.size] = pay
    if m:
        out[oi:oi + 4 * m] = np.concatenate(oidx).view(np.uint8)
        out[ov:ov + 4 * m] = np.concatenate(oval)
    out[tab:tab + 4 * table.size] = table.view(np.uint8)
    return out
