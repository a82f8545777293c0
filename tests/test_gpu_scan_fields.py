"""Fields just above 2048 groups of 8192 values: the smallest fields whose compress scans the
group sums in a single-workgroup kernel of its own instead of inside the compaction (prefixes
written once per super-group of 64 groups), through a plan with several lanes.

A batch of fields of different character (smooth, with escapes, constant so that it falls back to
a raw copy, special values, random bits) runs as launches of `lanes` fields and a ragged one,
then single calls on lane 0 (a synchronous compress, a capacity error reported in the result
record), then the batch again in the reverse order, for both coders. Every stream must equal the
oracle's ("Pipeline Specialization Internals", validation requirements: byte-identical compress)
and every reconstruction the oracle decoder's.
"""
import numpy as np
import pytest

import oracle
from error_bounded_lossy_encode_amd import synth
from helpers import CANARY, oracle_stream

pytestmark = pytest.mark.gpu

N = 2049 * 8192 + 333          # 2050 groups and a ragged tail
KINDS = ["smooth", "normal", "const", "specials", "bits"]


@pytest.fixture(scope="module")
def env():
    import torch
    from error_bounded_lossy_encode_amd import binding
    binding.lib()
    return binding, torch


def make_fields(seed, kinds):
    rng = np.random.default_rng(seed)
    fields = []
    for k, kind in enumerate(kinds):
        x = synth.tiny_array(rng, N, kind)
        if k == 1:
            x[::1001] = np.float32(np.inf)        # escapes
        fields.append(np.ascontiguousarray(x, dtype=np.float32))
    return fields


def check_streams(binding, oracle_refs, outs, recs, order):
    for slot, k in enumerate(order):
        ref = oracle_refs[k]
        nb, status = recs[slot]
        assert status == binding.EBLC_OK and nb == ref.size, (slot, k, nb, ref.size)
        got = outs[slot].cpu().numpy()
        assert np.array_equal(got[:nb], ref), f"field {k} (slot {slot}): stream differs"


@pytest.mark.parametrize("opts,lanes", [
    ("rel=1e-3;block=256;outlier_log2=15", 3),
    ("coder=chunk;chunk_bytes=8192;rel=1e-3;outlier_log2=15", 2),
])
def test_scan_kernel_fields_across_calls(env, opts, lanes):
    binding, torch = env
    kinds = KINDS if lanes == 3 else KINDS[:3]
    fields = make_fields(4242 + lanes, kinds)
    refs = [oracle_stream(oracle, f, [N], opts) for f in fields]
    assert int(refs[2][8]) == 1                   # the constant field falls back to a raw copy
    print(f"[scan-kernel fields] {opts} n={N} fields={len(fields)} lanes={lanes}", flush=True)
    st, plan = binding.eblc_plan_create([N], opts + f";lanes={lanes}", 0)
    assert st == binding.EBLC_OK, binding.eblc_status_string(st)
    try:
        maxb = binding.eblc_max_compressed_bytes(plan)
        xs = [torch.from_numpy(f).cuda() for f in fields]
        cnt = len(fields)
        outs = [torch.full((maxb + 32,), CANARY, dtype=torch.uint8, device="cuda") for _ in range(cnt)]
        res = torch.zeros(16 * cnt, dtype=torch.uint8, device="cuda")
        # 1. a batch: launches of `lanes` fields and a ragged one
        order = list(range(cnt))
        assert binding.eblc_compress_batch(plan, xs, outs, res, capacities=[maxb] * cnt) == binding.EBLC_OK
        check_streams(binding, refs, outs, binding.result_records(res), order)
        for o in outs:
            assert (o.cpu().numpy()[maxb:] == CANARY).all()
        ys = [torch.full((N,), float("nan"), dtype=torch.float32, device="cuda") for _ in range(cnt)]
        assert binding.eblc_decompress_batch(plan, outs, ys, [maxb] * cnt) == binding.EBLC_OK
        assert binding.eblc_plan_status(plan) == binding.EBLC_OK
        for k in range(cnt):
            _, ref_dec = oracle.decompress(refs[k])
            assert np.array_equal(ys[k].cpu().numpy().view(np.uint32), ref_dec.view(np.uint32)), k
        # 2. single calls on lane 0: a synchronous compress, then a capacity error, whose
        #    compaction writes nothing
        one = torch.full((maxb,), CANARY, dtype=torch.uint8, device="cuda")
        st, nb = binding.eblc_compress(plan, xs[1], one)
        assert st == binding.EBLC_OK and nb == refs[1].size
        assert np.array_equal(one.cpu().numpy()[:nb], refs[1])
        rec = torch.zeros(16, dtype=torch.uint8, device="cuda")
        small = torch.full((maxb,), CANARY, dtype=torch.uint8, device="cuda")
        cap = refs[0].size - 16
        assert binding.eblc_compress_async(plan, xs[0], small, rec, out_capacity=cap) == binding.EBLC_OK
        (nb, status), = binding.result_records(rec)
        assert status == binding.EBLC_CAPACITY and nb == refs[0].size
        assert (small.cpu().numpy()[cap:] == CANARY).all()
        # 3. the batch again in another order
        order = list(reversed(range(cnt)))
        for o in outs:
            o.fill_(CANARY)
        assert binding.eblc_compress_batch(plan, [xs[k] for k in order], outs, res,
                                           capacities=[maxb] * cnt) == binding.EBLC_OK
        check_streams(binding, refs, outs, binding.result_records(res), order)
        assert binding.eblc_plan_status(plan) == binding.EBLC_OK
    finally:
        binding.eblc_plan_destroy(plan)
