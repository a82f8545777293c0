"""Benchmark of the error-bounded float32 codec on one MI355X.

One step = compress every field of the workload, then decompress every stream (every stage of
the path), with the inputs already resident in HBM.  The default workload is the 512^3 float32
wavefield snapshot (eight Ricker wavelets, 40 % quiescent zeros) at relative bound 1e-3, block
256, outlier_log2 15.  Other workloads: c1 (2^20 sum of sines), c2 (4096^2 Gaussian random
field), c4 (2^28 AR(1) with 1 % spikes), c5_1e-6 / c5_1e-2 (64 snapshots of 256^3 compressed
back to back, then decompressed back to back).  By default the fields are compressed with
eblc_compress_batch (no host wait; lengths arrive in device result records) and decompressed
with eblc_decompress_batch and their buffers' capacity; a workload of several fields uses the
plan option lanes=8, which codes eight fields per kernel launch.  --api sync
uses eblc_compress, which waits once per field to return its length, and eblc_decompress.

Prints ONE JSON line: `value` is the round-trip throughput in GB/s of input bytes (input bytes
/ (compress + decompress time)); `compress_gbps`, `decompress_gbps` and `ratio` are given
separately; `roofline` is the encode kernel's achieved algorithmic bandwidth against the HBM
peak, from the mean duration of its launches in the timed steps (HIP event pairs the library
records around every launch, on the stream the launch runs on), with the rocprofv3-measured
traffic when a counter summary of the same kernel source exists under profiles/;
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, GB/s
METRIC = "compress/decompress GB/s (input bytes) at 1 MI355X, % of HBM peak; ratio"
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def build_items(name: str, device: str):
    """Returns ([(x device tensor, dims, options)], description)."""
    import torch

    from error_bounded_lossy_encode_amd import synth

    if name == "c1":
        xn, dims, opts = synth.c1_sines()
        return [(torch.from_numpy(xn).to(device), dims, opts)], \
            "1-D f32 n=2^20 sum of 4 sines + N(0,1e-3), abs eb 1e-3*range, block 32, T 15"
    if name == "c2":
        x, dims, opts = synth.c2_grf2d(4096, device=device)
        return [(x, dims, opts)], "2-D f32 4096x4096 Gaussian random field k^-3, rel eb 1e-2, block 128, T 15"
    if name == "c3":
        x, dims, opts = synth.c3_ricker(512, device=device)
        return [(x, dims, opts)], \
            "3-D f32 512^3 Ricker wavefield snapshot (8 sources, 40% zero), rel eb 1e-3, block 256, T 15"
    if name == "c4":
        xn, dims, opts = synth.c4_ar1_spikes()
        return [(torch.from_numpy(xn).to(device), dims, opts)], \
            "1-D f32 n=2^28 AR(1) phi 0.999 + 1% spikes, abs eb 1e-4*R, block 128, T 15, side_max 2^23"
    if name in ("c5_1e-6", "c5_1e-2"):
        rel = 1e-6 if name.endswith("1e-6") else 1e-2
        items = []
        for i in range(64):
            x, dims, opts = synth.c5_snapshot(i, 256, rel, device=device)
            items.append((x, dims, opts))
        return items, (f"64 x 3-D f32 256^3 Gaussian random fields k^-2 (seeds 100..163), rel eb {rel:g}, "
                       "block 256, T 30, compressed back to back then decompressed back to back")
    raise SystemExit(f"unknown workload {name}")


def parse_opts(opts: str, n: int) -> dict:
    """Options string -> the oracle's arguments (library defaults where absent); V is the chunk
    coder's chunk in values, None for the bitpack coder."""
    o = {"rel": True, "eps": 1e-4, "B": 256, "T": 30, "side_max": min(n, 1 << 23), "V": None, "center": False}
    for item in opts.split(";"):
        if "=" not in item:
            continue
        k, v = (s.strip() for s in item.split("="))
        if k in ("rel", "abs"):
            o["rel"], o["eps"] = k == "rel", float(v)
        elif k == "block":
            o["B"] = int(v)
        elif k == "outlier_log2":
            o["T"] = int(v)
        elif k == "side_max":
            o["side_max"] = int(v)
        elif k == "coder" and v == "chunk":
            o["V"] = o["V"] or 2048
        elif k == "chunk_bytes":
            o["V"] = int(v) // 4
        elif k == "center":
            o["center"] = v == "1"
    return o


def with_chunk_coder(opts: str, chunk_bytes: int) -> str:
    """A workload's options with its block replaced by the chunk coder."""
    items = [t for t in opts.split(";") if t.strip() and not t.strip().startswith("block=")]
    return ";".join(items + ["coder=chunk", f"chunk_bytes={chunk_bytes}"])


def host_cpu():
    """(CPU model, the host's logical cores, the threads this process may use): the cores it is
    pinned to, further limited by OMP_NUM_THREADS when that is set (a shared GPU host sets it to
    the CPU share of one GPU)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    total = os.cpu_count() or 1
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else total
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        usable = min(usable, int(omp))
    return model, total, max(1, usable)


def cpu_baseline(items, budget_s: float):
    """The oracle as it stands on a leading sample of the workload: whole fields while they fit
    the budget, else whole slowest-axis planes of the first field (the bound is resolved on the
    sample itself in relative mode).  It runs twice: single-threaded on the whole sample, then
    on P threads over P block-aligned pieces of it under the sample's bound (P = the threads the
    process may use, see host_cpu), whose joined stream must equal the single-threaded one.  A
    reported baseline, not a parity check of the GPU path."""
    import numpy as np

    import oracle
    from oracle import shards

    rate = 60e6  # values per second for compress + decompress together, a rough estimate
    budget_vals = budget_s * rate
    samples = []
    taken = 0
    for x, dims, opts in items:
        n = int(np.prod(dims))
        if taken + n <= budget_vals or not samples:
            if taken + n > budget_vals:  # first field too large: whole planes of it
                plane = int(np.prod(dims[1:])) if len(dims) > 1 else 1 << 16
                rows = max(1, int(budget_vals // plane))
                if len(dims) > 1:
                    rows = min(rows, dims[0])
                    sdims = [rows] + list(dims[1:])
                else:
                    rows = min(rows, n // plane)
                    sdims = [rows * plane]
                xs = x.reshape(-1)[: int(np.prod(sdims))].cpu().numpy()
                samples.append((xs, sdims, opts))
                taken += xs.size
                break
            samples.append((x.reshape(-1).cpu().numpy(), list(dims), opts))
            taken += n
        else:
            break
    model, host_cores, P = host_cpu()
    tc = td = pc = pd = 0.0
    nbytes = 0
    joined_ok = 0
    for xs, sdims, opts in samples:
        o = parse_opts(opts, xs.size)
        side_max = min(o["side_max"], xs.size)
        t0 = time.perf_counter()
        if o["V"] is not None:
            s = oracle.compress_chunked(xs, sdims, o["rel"], o["eps"], o["V"], o["T"], side_max)
        else:
            s = oracle.compress(xs, sdims, o["rel"], o["eps"], o["B"], o["T"], side_max, center=o["center"])
        t1 = time.perf_counter()
        st, y = oracle.decompress(s)
        t2 = time.perf_counter()
        assert st == oracle.OK
        ok, _, bounds, streams = shards.code_pieces(xs, o["rel"], o["eps"], o["B"], o["T"], o["center"],
                                                    o["V"], P, P)
        t3 = time.perf_counter()
        if ok:
            yp = shards.decode_pieces(streams, P)
        t4 = time.perf_counter()
        if ok:
            joined = shards.join(xs, sdims, o["T"], o["B"], side_max, o["center"], o["V"], bounds, streams)
            if joined is not None:
                assert np.array_equal(joined, s), "pieces do not join to the whole stream"
                assert np.array_equal(yp.view(np.uint32), y.view(np.uint32))
                joined_ok += 1
        tc += t1 - t0
        td += t2 - t1
        pc += t3 - t2
        pd += t4 - t3
        nbytes += 4 * xs.size
    return {
        "value": round(nbytes / (pc + pd) / 1e9, 4),
        "unit": "GB/s",
        "cores": P,
        "kind": "oracle",
        "host": {"cpu_model": model, "logical_cores": host_cores, "threads_used": P,
                 "note": "threads_used = the cores this process may use, limited by OMP_NUM_THREADS "
                         "(the CPU share of one GPU on a shared host)"},
        "sample": (f"{len(samples)} field(s), {taken} values ({nbytes / 2**20:.0f} MiB) from the start of the "
                   f"same workload, coded as {P} block-aligned pieces on {P} threads: compress "
                   f"{nbytes / pc / 1e9:.4f} GB/s, decompress {nbytes / pd / 1e9:.4f} GB/s (joined stream equal "
                   f"to the one-thread stream on {joined_ok} of {len(samples)} field(s)); one thread on the "
                   f"whole sample: compress {nbytes / tc / 1e9:.4f} GB/s, decompress {nbytes / td / 1e9:.4f} "
                   f"GB/s, round trip {nbytes / (tc + td) / 1e9:.4f} GB/s"),
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps; default: whole steps until at least 2 s have passed (at "
                         "least 10), since the GPU reaches its steady clocks only under sustained load")
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lanes", type=int, default=8,
                    help="plan option lanes=K for workloads of several fields: the batch calls code K "
                         "fields per kernel launch, each in its own workspace (the streams are the same "
                         "for every K)")
    ap.add_argument("--kernel-events", choices=["on", "off"], default="on",
                    help="on: the library records a HIP event pair around every encode and decode launch "
                         "of the timed steps (up to 8192 launches), for the rooflines")
    ap.add_argument("--event-every", type=int, default=4,
                    help="time the encode and decode launches of every k-th compress and decompress "
                         "launch sequence of the timed steps, and split every k-th step into its compress "
                         "and decompress time (each timed dispatch and each event costs the stream a few "
                         "microseconds)")
    ap.add_argument("--breakdown-steps", type=int, default=2,
                    help="untimed steps after the timed ones with an event pair around every launch, "
                         "for the per-kernel breakdown (event records delay the stream, so the timed "
                         "steps time only the two roofline kernels)")
    ap.add_argument("--api", choices=["batch", "sync"], default="batch",
                    help="batch: eblc_compress_batch (no host wait) and decompress by buffer capacity; "
                         "sync: eblc_compress per field, which waits to return each length")
    ap.add_argument("--halo", type=int, default=0, metavar="H",
                    help="store each field inside a buffer padded by H elements on every side of every "
                         "axis and compress / decompress through the padded strides")
    ap.add_argument("--coder", choices=["bitpack", "chunk"], default="bitpack",
                    help="bitpack: per-segment widths and fixed-length packing; chunk: the chunk-cooperative "
                         "coder (Quant, Diff, Bitshuffle, RZE)")
    ap.add_argument("--chunk-bytes", type=int, default=8192, choices=[4096, 8192, 16384])
    ap.add_argument("--center", action="store_true",
                    help="Lorenzo centering (bitpack coder): each block's first code against its mean")
    ap.add_argument("--extra-options", default="",
                    help="plan options appended to the workload's (e.g. lookback=0)")
    ap.add_argument("--cold-reps", type=int, default=3,
                    help="repetitions of the MALL-cold measurement (a 1 GiB device read before every "
                         "compress and decompress call); 0 skips it")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB device to device once (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the codec's multi-GPU "
              "sharding is a design note, not built", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from error_bounded_lossy_encode_amd import binding, profiling

    torch.cuda.set_device(0)
    dev = "cuda"
    log(f"[bench] generating workload {args.workload}")
    items, desc = build_items(args.workload, dev)
    items = [(x.contiguous(), dims, opts) for x, dims, opts in items]
    if args.center and args.coder == "chunk":
        raise SystemExit("--center applies to the bitpack coder only")
    if args.center:
        items = [(x, dims, opts + ";center=1") for x, dims, opts in items]
        desc += "; Lorenzo centering (block means)"
    if args.coder == "chunk":
        items = [(x, dims, with_chunk_coder(opts, args.chunk_bytes)) for x, dims, opts in items]
        desc = desc.replace(", block 128", "").replace(", block 256", "").replace(", block 32", "")
        desc += f"; chunk coder (Quant, Diff, Bitshuffle, RZE) over {args.chunk_bytes}-byte chunks"
    if args.extra_options:
        items = [(x, dims, opts + ";" + args.extra_options) for x, dims, opts in items]
        desc += f"; options {args.extra_options}"
    dims0, opts0 = items[0][1], items[0][2]
    assert all(d == dims0 and o == opts0 for _, d, o in items)
    n = items[0][0].numel()
    strides = None
    contiguous_items = items
    if args.halo > 0:
        # the solver's view: each field lives inside a halo-padded array
        h = args.halo
        pdims = [d + 2 * h for d in dims0]
        strides = [int(np.prod(pdims[a + 1:])) for a in range(len(pdims))]
        offset = sum(h * s for s in strides)
        span = 1 + sum((d - 1) * s for d, s in zip(dims0, strides))
        padded = []
        for x, dims, opts in items:
            buf = torch.zeros(offset + span + 4, dtype=torch.float32, device=dev)
            torch.as_strided(buf, dims0, strides, offset).copy_(x.reshape(dims0))
            padded.append((buf[offset:], dims, opts))
        items = padded
        desc += f"; stored with a {h}-element halo on every side (strides {strides})"
    plan_opts = opts0
    if len(items) > 1 and args.lanes > 1:
        plan_opts = opts0 + f";lanes={args.lanes}"
    log(f"[bench] {len(items)} field(s), n={n} dims={dims0} opts={plan_opts} strides={strides}")
    plan = binding.Plan(dims0, plan_opts, 0, strides=strides)
    outs = [torch.empty(plan.max_bytes, dtype=torch.uint8, device=dev) for _ in items]
    ys = [torch.empty_like(x) for x, _, _ in items]
    stream = torch.cuda.current_stream()
    nbytes = [plan.max_bytes] * len(items)
    xs = [x for x, _, _ in items]
    records = torch.zeros(16 * len(items), dtype=torch.uint8, device=dev)

    def compress_all():
        if args.api == "batch":
            st = binding.eblc_compress_batch(plan.handle, xs, outs, records, stream=stream)
            assert st == binding.EBLC_OK, binding.eblc_status_string(st)
            return
        for i, x in enumerate(xs):
            st, nb = binding.eblc_compress(plan.handle, x, outs[i], stream=stream)
            assert st == binding.EBLC_OK, binding.eblc_status_string(st)
            nbytes[i] = nb

    def decompress_all():
        # with the batch API the host never reads the lengths: each stream is decompressed with
        # its buffer's capacity and its own length comes from its header on the device
        if args.api == "batch":
            st = binding.eblc_decompress_batch(plan.handle, outs, ys, nbytes, stream=stream)
            assert st == binding.EBLC_OK, binding.eblc_status_string(st)
            return
        for i in range(len(items)):
            st = binding.eblc_decompress(plan.handle, outs[i], nbytes[i], ys[i], stream=stream)
            assert st == binding.EBLC_OK, binding.eblc_status_string(st)

    if args.warmup is not None:
        for _ in range(args.warmup):
            compress_all()
            decompress_all()
    else:
        args.warmup = 0
        t_w = time.perf_counter()
        while args.warmup < 10 or time.perf_counter() - t_w < 2.0:
            compress_all()
            decompress_all()
            args.warmup += 1
            if args.warmup % 10 == 0:
                torch.cuda.synchronize()
        log(f"[bench] {args.warmup} warmup steps")
    torch.cuda.synchronize()
    assert binding.eblc_plan_status(plan.handle) == binding.EBLC_OK

    # timed region: exactly K steps, bracketed by device syncs.  The library records an event
    # pair around each kernel launch of these steps on the stream it runs on (its own lane
    # streams included), up to 8192 launches: the per-kernel times below.
    # the compress / decompress split: event triples on every event_every-th step, one step
    # before those whose kernels the library times (so that the split holds no kernel events when
    # event_every > 1), and on the first step; the other steps carry no markers
    every = max(1, args.event_every)
    sampled = [k % every == (every - 2) % every or k == 0 for k in range(args.steps)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) if sampled[k] else None for k in range(args.steps)]
    timed_launches = min(8192, args.steps * len(items) * 2)
    if args.kernel_events == "on":
        assert binding.eblc_plan_set_profiling(plan.handle, timed_launches, "encode,decode",
                                               args.event_every) == binding.EBLC_OK
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if ev[k] is None:
            compress_all()
            decompress_all()
            continue
        ev[k][0].record(stream)
        compress_all()
        ev[k][1].record(stream)
        decompress_all()
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev = [e for e in ev if e is not None]
    assert binding.eblc_plan_status(plan.handle) == binding.EBLC_OK
    wall = (t1 - t0) / args.steps
    comp_ms = float(np.median([a.elapsed_time(b) for a, b, _ in ev]))
    decomp_ms = float(np.median([b.elapsed_time(c) for _, b, c in ev]))
    in_bytes = 4 * n * len(items)
    if args.api == "batch":
        recs = binding.result_records(records)
        assert all(status == binding.EBLC_OK for _, status in recs)
        nbytes = [nb for nb, _ in recs]
    total_stream = sum(nbytes)
    log(f"[bench] step {wall * 1e3:.3f} ms; compress {comp_ms:.3f} ms; decompress {decomp_ms:.3f} ms; "
        f"streams {total_stream} B")

    # roofline kernels: mean duration of encode and decode over their launches in the timed steps
    kavg, kcount = {}, {}
    if args.kernel_events == "on":
        for name, ms, cnt in binding.eblc_plan_kernel_times(plan.handle):
            kavg[name], kcount[name] = ms, cnt
        log("[bench] timed steps, kernel ms: " + ", ".join(f"{k}={v:.4f} (x{kcount[k]})" for k, v in kavg.items()))
    # breakdown of every kernel, from extra steps after the timed ones
    kall = {}
    if args.breakdown_steps > 0:
        assert binding.eblc_plan_set_profiling(plan.handle, min(8192, args.breakdown_steps * len(items) * 8)) \
            == binding.EBLC_OK
        for _ in range(args.breakdown_steps):
            compress_all()
            decompress_all()
        kall = {name: ms for name, ms, _ in binding.eblc_plan_kernel_times(plan.handle)}
        log("[bench] breakdown, kernel ms: " + ", ".join(f"{k}={v:.4f}" for k, v in kall.items()))
    binding.eblc_plan_set_profiling(plan.handle, 0)

    # MALL-cold figures: reading a 1 GiB buffer before every call evicts the 256 MB last-level
    # cache, so each call reads its input from HBM (fields up to 256 MB otherwise run from it).
    # The buffer is written once beforehand: a write before each call would leave dirty lines
    # whose write-back then overlaps the timed call.
    cold = None
    if args.cold_reps > 0:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.zeros(1, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        cc, cd = [], []
        for k in range(args.cold_reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            sink += flush.sum()
            e[0].record(stream)
            compress_all()
            e[1].record(stream)
            sink += flush.sum()
            e[2].record(stream)
            decompress_all()
            e[3].record(stream)
            torch.cuda.synchronize()
            cc.append(e[0].elapsed_time(e[1]))
            cd.append(e[2].elapsed_time(e[3]))
        del flush, sink
        assert binding.eblc_plan_status(plan.handle) == binding.EBLC_OK
        cold = {"compress_gbps": round(in_bytes / (float(np.median(cc)) * 1e-3) / 1e9, 3),
                "decompress_gbps": round(in_bytes / (float(np.median(cd)) * 1e-3) / 1e9, 3),
                "reps": args.cold_reps, "flush": "1 GiB device read before every compress and decompress call"}
        log(f"[bench] cold: compress {cold['compress_gbps']} GB/s, decompress {cold['decompress_gbps']} GB/s")

    # stream facts from the headers (host copies of 128 bytes, outside the timed region)
    nseg = (n + 31) // 32
    payload = []
    outliers = []
    ebs = []
    for i in range(len(items)):
        hdr = outs[i][:128].cpu().numpy()
        u64 = hdr.view(np.uint64)
        outliers.append(int(u64[9]))
        payload.append(int(u64[10]))
        ebs.append(float(hdr[56:60].view(np.float32)[0]))
        assert int(hdr[8]) == (2 if args.coder == "chunk" else 0), "stream fell back to RAW"
    # round-trip property, checked outside the timed region: every value within its own field's
    # bound (relative bounds differ from field to field)
    errs = []
    for i, (x, _, _) in enumerate(items):
        if strides is not None:
            xv = torch.as_strided(x, dims0, strides)
            yv = torch.as_strided(ys[i], dims0, strides)
        else:
            xv, yv = x, ys[i]
        fin = torch.isfinite(xv)
        e = float((yv - xv).abs()[fin].max())
        assert e <= ebs[i], f"field {i}: max |x - x'| {e} above its eb {ebs[i]}"
        errs.append(e)
    err_max = max(errs)
    wi = max(range(len(items)), key=lambda i: errs[i] / ebs[i] if ebs[i] > 0 else 0.0)
    log(f"[bench] {len(items)} field(s) within their own bounds; closest, field {wi}: eb={ebs[wi]:.6g} "
        f"max|x-x'|={errs[wi]:.6g}; outliers(first)={outliers[0]}")

    # algorithmic bytes per launch: encode reads 4n and writes the size section (a width byte per
    # segment, or a u32 word count per chunk) and the payload words; decode reads them and writes 4n
    avg_payload = float(np.mean(payload))
    if args.coder == "chunk":
        V = args.chunk_bytes // 4
        sizes = 4 * ((n + V - 1) // V)
        kernels = ("chunk_encode_kernel", "chunk_decode_kernel")
        tag = f"{args.workload}_chunk{args.chunk_bytes}"
    else:
        sizes = nseg
        kernels = ("encode_kernel", "decode_kernel")
        tag = args.workload
        if args.center:
            B = int(parse_opts(opts0, n)["B"])
            sizes += 4 * ((n + B - 1) // B)   # the means stream
            tag += "_center"
    enc_bytes = 4 * n + sizes + avg_payload
    dec_bytes = sizes + avg_payload + 4 * n
    # a launch codes up to `lanes` fields: the fields of a step over the launches of a stage
    lanes = args.lanes if len(items) > 1 and args.api == "batch" else 1
    per_launch = len(items) / -(-len(items) // lanes)
    # a counter summary holds for its own launch configuration only
    if args.halo > 0:
        tag += f"_halo{args.halo}"
    if len(items) > 1:
        tag += f"_x{per_launch:g}"
    traffic = profiling.read_traffic(os.path.join(PROFILES, f"traffic_{tag}.txt"))

    # whole-call fractions of the HBM peak: algorithmic bytes (compress reads the field, twice in
    # relative mode, and writes the streams; decompress reads the streams, writes the field, and
    # the outlier patch reads 8 and writes 4 bytes per outlier) over the call time, and the
    # counter-measured bytes of every kernel of the call, when the traffic summary matches
    rel_mode = bool(parse_opts(opts0, n)["rel"])
    total_m = int(sum(outliers))
    comp_alg = in_bytes * (2 if rel_mode else 1) + total_stream
    decomp_alg = total_stream + in_bytes + 12 * total_m
    launches_per_stage = -(-len(items) // lanes)
    # a field of at most 2048 groups of 8192 values scans its group sums inside the compaction
    tail = ("compact_scan_kernel",) if -(-n // 8192) <= 2048 else ("scan_compress_kernel", "compact_kernel")
    comp_kernels = ("range_partial_kernel", "range_resolve_kernel", kernels[0]) + tail
    dec_kernels = (kernels[1], "patch_kernel")

    def call_frac(alg, ms, ks):
        secs = ms * 1e-3
        out = {"alg_bytes": int(alg), "ms": round(ms, 4), "hbm_frac": round(alg / secs / 1e9 / HBM_PEAK_GBPS, 4),
               "traffic_bytes": None, "traffic_frac": None}
        if traffic is not None and all(k in traffic for k in ks if k != "range_partial_kernel"
                                       and k != "range_resolve_kernel"):
            tb = launches_per_stage * sum(traffic.get(k, 0.0) for k in ks)
            out["traffic_bytes"] = int(tb)
            out["traffic_frac"] = round(tb / secs / 1e9 / HBM_PEAK_GBPS, 4)
        return out

    whole_call = {"compress": call_frac(comp_alg, comp_ms, comp_kernels),
                  "decompress": call_frac(decomp_alg, decomp_ms, dec_kernels),
                  "note": "algorithmic: compress 4n read (+4n range read in relative mode) + stream written; "
                          "decompress stream read + 4n written + 12 B per outlier; traffic: rocprofv3 "
                          "FETCH_SIZE + WRITE_SIZE of every kernel of the call, scaled by a plain copy"}

    def roof(name, alg_bytes, key):
        # algorithmic bytes per launch over the mean launch duration in the timed steps
        if key not in kavg:
            return None
        achieved = per_launch * alg_bytes / (kavg[key] * 1e-3) / 1e9
        t = None if traffic is None else traffic.get(name)
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None if t is None else round(t),
                "kernel": name, "launches": kcount[key]}

    result = {
        "metric": METRIC,
        "value": round(in_bytes / wall / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": desc, "fields": len(items), "n": n, "dims": dims0, "options": opts0,
                   "strides": strides, "lanes": args.lanes if len(items) > 1 else 1,
                   "step": "compress all fields, then decompress all streams",
                   "api": "eblc_compress_batch + eblc_decompress_batch" if args.api == "batch"
                   else "eblc_compress (waits per field) + eblc_decompress"},
        "compress_gbps": round(in_bytes / (comp_ms * 1e-3) / 1e9, 3),
        "decompress_gbps": round(in_bytes / (decomp_ms * 1e-3) / 1e9, 3),
        "compress_hbm_frac": whole_call["compress"]["hbm_frac"],
        "decompress_hbm_frac": whole_call["decompress"]["hbm_frac"],
        "whole_call": whole_call,
        "ratio": round(in_bytes / total_stream, 4),
        "compressed_bytes": total_stream,
        "outliers": int(sum(outliers)),
        "kernel_ms": {k: round(v, 5) for k, v in kall.items()},
        "kernel_ms_note": "every kernel, event pairs in untimed steps after the timed ones; the rooflines use "
                          "encode and decode launches timed inside the timed steps",
        "roofline": roof(kernels[0], enc_bytes, "encode"),
        "roofline_decode": roof(kernels[1], dec_bytes, "decode"),
        "algorithmic_bytes_per_launch": {"encode": round(per_launch * enc_bytes), "decode": round(per_launch * dec_bytes)},
        "fields_per_launch": per_launch,
        "cold": cold,
        "max_abs_err": err_max,
        "eb": ebs[0],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(contiguous_items, args.cpu_budget)
    plan.close()
    if args.calibrate_copy > 0:
        # a plain device-to-device copy of known size, for scaling the HBM byte counters
        nb = args.calibrate_copy << 20
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {nb} bytes done")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
