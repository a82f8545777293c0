"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Streams must be byte-identical (header, widths, payload words, outliers, pads) and the
GPU reconstruction bit-identical to the oracle's decoder, on seeded inputs that span several
chunks and end in a ragged tail, for every block size, both bound modes and the RAW fallbacks.
"""
import numpy as np
import pytest

import oracle
from error_bounded_lossy_encode_amd import synth
from helpers import first_difference, gpu_roundtrip, header, oracle_stream, parse_options

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    from error_bounded_lossy_encode_amd import binding
    binding.lib()
    return binding, torch


def check_case(env, x, dims, opts, label=""):
    binding, torch = env
    n = int(np.prod(dims))
    o = parse_options(opts, n)
    ref = oracle.compress(x, dims, o["rel"], o["eps"], o["B"], o["T"], o["side_max"])
    st, ref_dec = oracle.decompress(ref)
    assert st == oracle.OK
    got, dec = gpu_roundtrip(binding, torch, x, dims, opts)
    assert got.size == ref.size and np.array_equal(got, ref), \
        f"{label} {opts}: {first_difference(got, ref)}"
    assert np.array_equal(dec.view(np.uint32), ref_dec.view(np.uint32)), \
        f"{label} {opts}: reconstruction differs at {np.nonzero(dec.view(np.uint32) != ref_dec.view(np.uint32))[0][:5]}"
    return header(ref)


@pytest.mark.parametrize("seed", range(6))
def test_tiny_fuzz(env, seed):
    rng = np.random.default_rng(500 + seed)
    kinds = ["smooth", "normal", "specials", "const", "ramp", "subnormal", "bits"]
    for case in range(20):
        n = int(rng.integers(1, 301))
        kind = kinds[(seed + case) % len(kinds)]
        x = synth.tiny_array(rng, n, kind)
        B = int(rng.choice([32, 64, 96, 128, 160, 256, 480, 512, 992, 1024, 2048]))
        T = int(rng.choice([1, 2, 15, 30]))
        side = int(rng.choice([0, 1, n]))
        if rng.integers(0, 2):
            eps = float(rng.choice([0.0, 1e-7, 1e-3, 0.3]))
            opts = f"rel={eps!r};block={B};outlier_log2={T};side_max={side}"
        else:
            eps = float(rng.choice([0.0, 1e-6, 1e-2, 5.0]))
            opts = f"abs={eps!r};block={B};outlier_log2={T};side_max={side}"
        check_case(env, x, [n], opts, f"seed{seed} case{case} {kind} n={n}")


@pytest.mark.parametrize("B", [32, 64, 128, 256, 512, 1024, 2048])
def test_multichunk_ragged(env, B):
    rng = np.random.default_rng(B)
    for n in [2048, 2049, 3 * 2048 + 777, 4 * 4 * 2048 + 5, (1 << 17) + 1234]:
        for kind in ["smooth", "specials"]:
            x = synth.tiny_array(rng, n, kind)
            check_case(env, x, [n], f"rel=1e-3;block={B};outlier_log2=15", f"{kind} n={n}")
        x = synth.tiny_array(rng, n, "normal")
        check_case(env, x, [n], f"abs=0.01;block={B};outlier_log2=30", f"normal n={n}")


def test_wide_codes_and_escapes(env):
    """Widths up to 32 (T = 30, tiny bound) and many escapes (T small) across chunks."""
    rng = np.random.default_rng(77)
    n = 5 * 2048 + 333
    x = (rng.normal(0, 1, n) * 1e3).astype(np.float32)
    check_case(env, x, [n], "abs=1e-5;block=256;outlier_log2=30", "wide")
    check_case(env, x, [n], "abs=1e-2;block=64;outlier_log2=8", "escapes")
    xs = x.copy()
    xs[rng.integers(0, n, 300)] = np.float32(np.nan)
    check_case(env, xs, [n], "rel=1e-4;block=128;outlier_log2=15", "nan escapes")


def test_multidim_shapes(env):
    rng = np.random.default_rng(3)
    for dims in ([33, 65], [7, 9, 300], [2, 3, 4, 1000]):
        n = int(np.prod(dims))
        x = synth.tiny_array(rng, n, "smooth")
        check_case(env, x, dims, "rel=1e-3;block=128", f"dims={dims}")


def test_small_configs(env):
    """The five workloads at sizes the oracle finishes in seconds."""
    x, dims, opts = synth.c1_sines(1 << 20)
    check_case(env, x, dims, opts, "C1 full")
    x, dims, opts = synth.c2_grf2d(512)
    check_case(env, x.numpy(), dims, opts, "C2 512^2")
    x, dims, opts = synth.c3_ricker(96)
    check_case(env, x.numpy(), dims, opts, "C3 96^3")
    x, dims, opts = synth.c4_ar1_spikes(1 << 20, side_max=1 << 15)
    h = check_case(env, x, dims, opts, "C4 2^20")
    assert h["mode"] == 0 and h["m"] > 5000
    for rel in (1e-6, 1e-2):
        x, dims, opts = synth.c5_snapshot(0, 48, rel)
        check_case(env, x.numpy(), dims, opts, f"C5 48^3 rel={rel}")


GENERAL_BLOCKS = [96, 160, 480, 992]


def check_any(env, x, dims, opts, label=""):
    """check_case for any options string (centering included)."""
    binding, torch = env
    ref = oracle_stream(oracle, x, dims, opts)
    st, ref_dec = oracle.decompress(ref)
    assert st == oracle.OK
    got, dec = gpu_roundtrip(binding, torch, x, dims, opts)
    assert got.size == ref.size and np.array_equal(got, ref), f"{label} {opts}: {first_difference(got, ref)}"
    bad = np.nonzero(dec.view(np.uint32) != ref_dec.view(np.uint32))[0]
    assert bad.size == 0, f"{label} {opts}: reconstruction differs at {bad[:5]}"
    return header(ref)


@pytest.mark.parametrize("B", GENERAL_BLOCKS)
def test_general_blocks_ragged(env, B):
    """Blocks that are multiples of 32 but not powers of two ("Pipeline Specialization
    Internals", Forward declaration: the block is a multiple of 32): blocks then start inside
    encode and decode chunks and cross their ends.  Ragged lengths over several workgroups,
    both bound modes, escapes, and centering, whose means may need codes of the next chunk."""
    rng = np.random.default_rng(900 + B)
    for n in [B - 27, B + 1, 2049, 3 * 2048 + 777, 4 * 4 * 2048 + 5, (1 << 17) + 1234]:
        for kind in ["smooth", "specials"]:
            x = synth.tiny_array(rng, n, kind)
            check_any(env, x, [n], f"rel=1e-3;block={B};outlier_log2=15", f"{kind} n={n}")
            x = (x + np.float32(25.0)).astype(np.float32)
            check_any(env, x, [n], f"rel=1e-4;block={B};outlier_log2=30;center=1", f"centered {kind} n={n}")
        x = synth.tiny_array(rng, n, "normal")
        check_any(env, x, [n], f"abs=0.01;block={B};outlier_log2=30", f"normal n={n}")
        x = synth.tiny_array(rng, n, "smooth")
        x[5::29] = np.float32(1e9)                # more than 64 escapes per chunk
        check_any(env, x, [n], f"abs=0.01;block={B};outlier_log2=30;center=1", f"escapes n={n}")


def test_general_blocks_decode_across_plans(env):
    """A stream decodes with the block recorded in it, whichever block the decoding plan has:
    streams of blocks that are not powers of two through a plan of block 256, and the reverse."""
    binding, torch = env
    rng = np.random.default_rng(31)
    n = 3 * 8192 + 517
    x = (synth.tiny_array(rng, n, "smooth") + np.float32(9.0)).astype(np.float32)
    cases = [("rel=1e-3;block=96;outlier_log2=15", "rel=1e-3;block=256"),
             ("rel=1e-3;block=480;center=1", "rel=1e-3;block=256"),
             ("rel=1e-3;block=256;center=1", "rel=1e-3;block=160"),
             ("rel=1e-3;block=2048", "rel=1e-3;block=992;center=1")]
    for enc_opts, dec_opts in cases:
        ref = oracle_stream(oracle, x, [n], enc_opts)
        _, ref_dec = oracle.decompress(ref)
        st, plan = binding.eblc_plan_create([n], dec_opts, 0)
        assert st == binding.EBLC_OK
        try:
            stream = torch.from_numpy(ref).cuda()
            y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
            assert binding.eblc_decompress(plan, stream, ref.size, y) == binding.EBLC_OK
            assert binding.eblc_plan_status(plan) == binding.EBLC_OK, (enc_opts, dec_opts)
            assert np.array_equal(y.cpu().numpy().view(np.uint32), ref_dec.view(np.uint32)), (enc_opts, dec_opts)
        finally:
            binding.eblc_plan_destroy(plan)
