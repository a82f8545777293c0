"""Test helpers: option parsing for the oracle, GPU round trips through the C ABI, stream
comparison with section-level diagnostics."""
from __future__ import annotations

import numpy as np

CANARY = 0xA7


def parse_options(opts: str, n: int):
    """Options string -> oracle arguments (rel, eps, B, T, side_max, V), library defaults.
    V is the chunk coder's chunk in values (coder=chunk), else None."""
    out = {"rel": True, "eps": 1e-4, "B": 256, "T": 30, "side_max": min(n, 1 << 23), "V": None,
           "center": False}
    if opts is None or opts.strip() == "":
        return out
    try:
        out["eps"] = float(opts)
        return out
    except ValueError:
        pass
    for item in opts.split(";"):
        item = item.strip()
        if not item:
            continue
        k, v = item.split("=")
        k, v = k.strip(), v.strip()
        if k in ("rel", "abs"):
            out["rel"] = k == "rel"
            out["eps"] = float(v)
        elif k == "block":
            out["B"] = int(v)
        elif k == "outlier_log2":
            out["T"] = int(v)
        elif k == "side_max":
            out["side_max"] = int(v)
        elif k == "coder" and v == "chunk":
            out["V"] = out["V"] or 2048
        elif k == "chunk_bytes":
            out["V"] = int(v) // 4
        elif k == "center":
            out["center"] = v == "1"
    return out


def chunk_options(opts: str, chunk_bytes: int) -> str:
    """A workload's options with its block replaced by the chunk coder of chunk_bytes."""
    items = [t for t in opts.split(";") if t.strip() and not t.strip().startswith("block=")]
    return ";".join(items + ["coder=chunk", f"chunk_bytes={chunk_bytes}"])


def oracle_stream(oracle, x: np.ndarray, dims, opts: str) -> np.ndarray:
    """The oracle's stream for the library's options string (either coder)."""
    n = int(np.prod(dims))
    o = parse_options(opts, n)
    if o["V"] is not None:
        return oracle.compress_chunked(x, dims, o["rel"], o["eps"], o["V"], o["T"], o["side_max"])
    return oracle.compress(x, dims, o["rel"], o["eps"], o["B"], o["T"], o["side_max"], center=o["center"])


def header(stream: np.ndarray) -> dict:
    b = np.ascontiguousarray(stream[:128])
    u32 = b.view(np.uint32)
    u64 = b.view(np.uint64)
    return {"mode": int(b[8]), "n": int(u64[6]), "eb_f_bits": int(u32[14]), "m": int(u64[9]),
            "payload_bytes": int(u64[10]), "payload_off": int(u64[12]), "oidx_off": int(u64[13]),
            "oval_off": int(u64[14]), "total": int(u64[15])}


def first_difference(a: np.ndarray, b: np.ndarray) -> str:
    """Describe where two streams first differ, by section."""
    if a.size != b.size:
        msg = f"length {a.size} vs {b.size}; "
    else:
        msg = ""
    m = min(a.size, b.size)
    diff = np.nonzero(a[:m] != b[:m])[0]
    if diff.size == 0:
        return msg + "common prefix identical"
    i = int(diff[0])
    h = header(b) if b.size >= 128 else None
    sec = "header"
    if h is not None and i >= 128:
        sec = "widths"
        for name, off in (("payload", h["payload_off"]), ("outlier idx", h["oidx_off"]),
                          ("outlier val", h["oval_off"])):
            if i >= off:
                sec = name
    return msg + f"first differing byte {i} ({sec}), {diff.size} bytes differ"


def gpu_roundtrip(binding, torch, x_np: np.ndarray, dims, opts: str, canary: int = 64,
                  stream=None, out_capacity=None):
    """Compress on the GPU and decompress the result; returns (stream bytes, decoded floats)."""
    n = int(np.prod(dims))
    st, plan = binding.eblc_plan_create(dims, opts, 0)
    assert st == binding.EBLC_OK, binding.eblc_status_string(st)
    try:
        maxb = binding.eblc_max_compressed_bytes(plan)
        x = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
        out = torch.full((maxb + canary,), CANARY, dtype=torch.uint8, device="cuda")
        st, nbytes = binding.eblc_compress(plan, x, out, maxb if out_capacity is None else out_capacity,
                                           stream=stream)
        assert st == binding.EBLC_OK, binding.eblc_status_string(st)
        host = out.cpu().numpy()
        assert (host[nbytes:] == CANARY).all() if out_capacity is None else True, "write past the stream"
        y = torch.full((n + 16,), float("nan"), dtype=torch.float32, device="cuda")
        st = binding.eblc_decompress(plan, out, nbytes, y, stream=stream)
        assert st == binding.EBLC_OK, binding.eblc_status_string(st)
        st = binding.eblc_plan_status(plan, stream=stream)
        assert st == binding.EBLC_OK, binding.eblc_status_string(st)
        yh = y.cpu().numpy()
        assert np.isnan(yh[n:]).all(), "decoder wrote past n"
        return host[:nbytes].copy(), yh[:n].copy()
    finally:
        binding.eblc_plan_destroy(plan)


def oracle_threads() -> int:
    """Threads for the sharded oracle: the host's cores, at most 16 (a GPU machine's CPU share)."""
    import os
    return max(1, min(16, os.cpu_count() or 1))


def oracle_reference(oracle, shards, x: np.ndarray, dims, opts: str, threads: int | None = None):
    """The oracle's stream and reconstruction for a full-size field, coded as block-aligned
    pieces on several threads and joined (the join reproduces the whole-field stream byte for
    byte; it is pinned against the one-thread oracle in test_oracle_shards.py).  A stream that
    falls back to a raw copy is made by the one-thread oracle instead."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    n = int(np.prod(dims))
    o = parse_options(opts, n)
    threads = threads or oracle_threads()
    ok, _, bounds, streams = shards.code_pieces(x, o["rel"], o["eps"], o["B"], o["T"], o["center"], o["V"],
                                                threads, threads)
    if ok:
        joined = shards.join(x, dims, o["T"], o["B"], o["side_max"], o["center"], o["V"], bounds, streams)
        if joined is not None and int(joined[8]) != 1:
            return joined, shards.decode_pieces(streams, threads)
    ref = oracle_stream(oracle, x, dims, opts)
    st, y = oracle.decompress(ref)
    assert st == oracle.OK
    return ref, y
