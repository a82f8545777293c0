"""The asynchronous and batched compress entry points against the oracle.

The result record arrives in device memory or pinned host memory; streams are decompressed
with the buffer's capacity instead of their length (the length is read from the stream's header
on the device), so the host never waits between compress and decompress.
"""
import numpy as np
import pytest

import oracle
from error_bounded_lossy_encode_amd import synth
from helpers import CANARY, parse_options

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    from error_bounded_lossy_encode_amd import binding
    binding.lib()
    return binding, torch


def oracle_stream(x, dims, opts):
    o = parse_options(opts, x.size)
    return oracle.compress(x, dims, o["rel"], o["eps"], o["B"], o["T"], o["side_max"])


@pytest.mark.parametrize("where", ["device", "pinned"])
def test_async_compress_then_decompress_without_host_wait(env, where):
    binding, torch = env
    rng = np.random.default_rng(31)
    n = 7 * 2048 + 123
    x = synth.tiny_array(rng, n, "smooth")
    x[::997] = np.float32(np.nan)
    dims, opts = [n], "rel=1e-4;block=256;outlier_log2=15"
    ref = oracle_stream(x, dims, opts)
    st, plan = binding.eblc_plan_create(dims, opts, 0)
    assert st == binding.EBLC_OK
    try:
        maxb = binding.eblc_max_compressed_bytes(plan)
        xd = torch.from_numpy(x).cuda()
        out = torch.full((maxb + 64,), CANARY, dtype=torch.uint8, device="cuda")
        if where == "device":
            res = torch.zeros(16, dtype=torch.uint8, device="cuda")
        else:
            res = torch.zeros(16, dtype=torch.uint8).pin_memory()
        y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        assert binding.eblc_compress_async(plan, xd, out, res, out_capacity=maxb) == binding.EBLC_OK
        assert binding.eblc_decompress(plan, out, maxb, y) == binding.EBLC_OK
        assert binding.eblc_plan_status(plan) == binding.EBLC_OK
        (nb, status), = binding.result_records(res)
        assert status == binding.EBLC_OK and nb == ref.size
        got = out.cpu().numpy()
        assert np.array_equal(got[:nb], ref) and (got[maxb:] == CANARY).all()
        st, ref_dec = oracle.decompress(ref)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref_dec.view(np.uint32))
    finally:
        binding.eblc_plan_destroy(plan)


def test_async_capacity_error_in_record(env):
    binding, torch = env
    rng = np.random.default_rng(5)
    n = 3 * 2048 + 9
    x = (rng.normal(0, 1, n)).astype(np.float32)
    dims, opts = [n], "abs=1e-6;block=64;outlier_log2=30"
    ref = oracle_stream(x, dims, opts)
    st, plan = binding.eblc_plan_create(dims, opts, 0)
    try:
        maxb = binding.eblc_max_compressed_bytes(plan)
        xd = torch.from_numpy(x).cuda()
        out = torch.full((maxb,), CANARY, dtype=torch.uint8, device="cuda")
        res = torch.zeros(16, dtype=torch.uint8, device="cuda")
        cap = ref.size - 48
        assert binding.eblc_compress_async(plan, xd, out, res, out_capacity=cap) == binding.EBLC_OK
        (nb, status), = binding.result_records(res)
        assert status == binding.EBLC_CAPACITY and nb == ref.size
        assert (out.cpu().numpy()[cap:] == CANARY).all()
        # misaligned record pointer is refused before anything is enqueued
        assert binding.lib().eblc_compress_async(plan, xd.data_ptr(), out.data_ptr(), maxb,
                                                 res.data_ptr() + 4, None) == binding.EBLC_INVALID_ARGUMENT
    finally:
        binding.eblc_plan_destroy(plan)


@pytest.mark.parametrize("lanes,dec", [(1, "loop"), (1, "batch"), (3, "loop"), (3, "batch"), (8, "batch")])
def test_batch_of_fields(env, lanes, dec):
    """Snapshots of different character through one plan, then decompressed; every stream and
    reconstruction matches the oracle's, whether the fields run one per launch (one lane) or
    several per launch, each in its own lane's workspace."""
    binding, torch = env
    N = 40
    dims, opts = [N, N, N], "rel=1e-3;block=256;outlier_log2=15"
    plan_opts = opts + f";lanes={lanes}"
    fields = []
    for i in range(6):
        x, _, _ = synth.c5_snapshot(i, N, 1e-3)
        x = x.numpy().copy()
        if i == 2:
            x[:: 101] = np.float32(np.inf)          # escapes
        if i == 4:
            x[:] = np.float32(3.0)                  # constant field: bound unusable -> RAW
        fields.append(x)
    st, plan = binding.eblc_plan_create(dims, plan_opts, 0)
    assert st == binding.EBLC_OK
    try:
        maxb = binding.eblc_max_compressed_bytes(plan)
        xs = [torch.from_numpy(f).cuda() for f in fields]
        outs = [torch.full((maxb,), CANARY, dtype=torch.uint8, device="cuda") for _ in fields]
        res = torch.zeros(16 * len(fields), dtype=torch.uint8, device="cuda")
        ys = [torch.full((N ** 3,), float("nan"), dtype=torch.float32, device="cuda") for _ in fields]
        assert binding.eblc_compress_batch(plan, xs, outs, res) == binding.EBLC_OK
        if dec == "batch":
            assert binding.eblc_decompress_batch(plan, outs, ys, [maxb] * len(fields)) == binding.EBLC_OK
        else:
            for i in range(len(fields)):
                assert binding.eblc_decompress(plan, outs[i], maxb, ys[i]) == binding.EBLC_OK
        # no host wait before reading: the copies below follow the batch on the caller's stream
        ycopy = [y.clone() for y in ys]
        assert binding.eblc_plan_status(plan) == binding.EBLC_OK
        recs = binding.result_records(res)
        for i, f in enumerate(fields):
            ref = oracle_stream(f, dims, opts)
            nb, status = recs[i]
            assert status == binding.EBLC_OK and nb == ref.size, i
            assert np.array_equal(outs[i].cpu().numpy()[:nb], ref), i
            _, ref_dec = oracle.decompress(ref)
            assert np.array_equal(ycopy[i].cpu().numpy().view(np.uint32), ref_dec.view(np.uint32)), i
        assert int(outs[4].cpu().numpy()[8]) == 1  # the constant field went RAW
        assert binding.eblc_compress_batch(plan, [], [], res) == binding.EBLC_OK
        assert binding.eblc_decompress_batch(plan, [], []) == binding.EBLC_OK
    finally:
        binding.eblc_plan_destroy(plan)


def test_batch_lanes_report_corrupt_stream_of_any_lane(env):
    """A corrupt stream decoded on a lane other than the first sets the plan's sticky status,
    which eblc_plan_status returns once and then clears; the other streams still decode."""
    binding, torch = env
    N = 32
    dims, opts = [N, N, N], "rel=1e-3;block=256;outlier_log2=15;lanes=4"
    st, plan = binding.eblc_plan_create(dims, opts, 0)
    assert st == binding.EBLC_OK
    try:
        maxb = binding.eblc_max_compressed_bytes(plan)
        fields = [synth.c5_snapshot(i, N, 1e-3)[0].numpy().copy() for i in range(6)]
        xs = [torch.from_numpy(f).cuda() for f in fields]
        outs = [torch.zeros((maxb,), dtype=torch.uint8, device="cuda") for _ in fields]
        res = torch.zeros(16 * len(fields), dtype=torch.uint8, device="cuda")
        assert binding.eblc_compress_batch(plan, xs, outs, res) == binding.EBLC_OK
        outs[5][0] ^= 0xFF                      # field 5 is lane 1 of the second group: bad magic
        ys = [torch.zeros((N ** 3,), dtype=torch.float32, device="cuda") for _ in fields]
        assert binding.eblc_decompress_batch(plan, outs, ys) == binding.EBLC_OK
        assert binding.eblc_plan_status(plan) == binding.EBLC_CORRUPT_STREAM
        assert binding.eblc_plan_status(plan) == binding.EBLC_OK
        for i in range(5):
            _, ref_dec = oracle.decompress(oracle_stream(fields[i], dims, opts.rsplit(";", 1)[0]))
            assert np.array_equal(ys[i].cpu().numpy().view(np.uint32), ref_dec.view(np.uint32)), i
        # arguments are checked before anything is enqueued
        bad = [outs[0], outs[1]]
        assert binding.eblc_decompress_batch(plan, bad, ys[:2], [maxb, 64]) == binding.EBLC_CORRUPT_STREAM
    finally:
        binding.eblc_plan_destroy(plan)


def test_kernel_time_records_cover_every_lane(env):
    """The measurement hook records every launch of a batch (one per stage for each group of
    `lanes` fields) and folds the records by kernel name."""
    binding, torch = env
    N = 32
    dims = [N, N, N]
    st, plan = binding.eblc_plan_create(dims, "rel=1e-3;lanes=3", 0)
    assert st == binding.EBLC_OK
    try:
        maxb = binding.eblc_max_compressed_bytes(plan)
        xs = [synth.c5_snapshot(i, N, 1e-3)[0].cuda() for i in range(5)]
        outs = [torch.zeros((maxb,), dtype=torch.uint8, device="cuda") for _ in xs]
        ys = [torch.zeros((N ** 3,), dtype=torch.float32, device="cuda") for _ in xs]
        res = torch.zeros(16 * len(xs), dtype=torch.uint8, device="cuda")
        assert binding.eblc_plan_set_profiling(plan, 1000) == binding.EBLC_OK
        assert binding.eblc_compress_batch(plan, xs, outs, res) == binding.EBLC_OK
        assert binding.eblc_decompress_batch(plan, outs, ys) == binding.EBLC_OK
        rec = binding.eblc_plan_kernel_times(plan)
        names = [r[0] for r in rec]
        # a field of at most 2048 groups scans its group sums inside the compaction
        assert names == ["range", "encode", "compact", "decode", "patch"]
        assert all(cnt == 2 and ms > 0 for _, ms, cnt in rec)  # groups of 3 and 2 fields
        assert binding.eblc_plan_kernel_times(plan) == []       # records cleared by the read
        assert binding.eblc_plan_set_profiling(plan, 3) == binding.EBLC_OK
        assert binding.eblc_compress_batch(plan, xs, outs, res) == binding.EBLC_OK
        assert sum(cnt for _, _, cnt in binding.eblc_plan_kernel_times(plan)) == 3  # pool of 3 launches
        # only the named kernels are timed
        assert binding.eblc_plan_set_profiling(plan, 1000, "decode,encode") == binding.EBLC_OK
        assert binding.eblc_compress_batch(plan, xs, outs, res) == binding.EBLC_OK
        assert binding.eblc_decompress_batch(plan, outs, ys) == binding.EBLC_OK
        rec = binding.eblc_plan_kernel_times(plan)
        assert [(r[0], r[2]) for r in rec] == [("encode", 2), ("decode", 2)]
        # sampled: every second launch sequence of each kind (two batches of two groups each)
        assert binding.eblc_plan_set_profiling(plan, 1000, "encode,decode", 2) == binding.EBLC_OK
        for _ in range(2):
            assert binding.eblc_compress_batch(plan, xs, outs, res) == binding.EBLC_OK
            assert binding.eblc_decompress_batch(plan, outs, ys) == binding.EBLC_OK
        rec = binding.eblc_plan_kernel_times(plan)
        assert [(r[0], r[2]) for r in rec] == [("encode", 2), ("decode", 2)]
        assert binding.eblc_plan_set_profiling(plan, 10, None, 0) == binding.EBLC_INVALID_ARGUMENT
        assert binding.eblc_plan_set_profiling(plan, 0) == binding.EBLC_OK
        with pytest.raises(RuntimeError):
            binding.eblc_plan_kernel_times(plan)
        assert binding.eblc_plan_status(plan) == binding.EBLC_OK
    finally:
        binding.eblc_plan_destroy(plan)
