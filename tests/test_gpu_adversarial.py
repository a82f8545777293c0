"""The quantizer's hard cases on the GPU, against the oracle.

Fields of several encode workgroups with ragged tails are filled with values placed where the
verified quantizer must decide carefully ("Pipeline Specialization Internals", linear
quantization with step 2*eb): cell boundaries (k + 1/2) s, grid points, +-eb and values within a
millionth of it (codes +-1 beside the bound, where the exactness clause |x| >= |y|/2 matters),
codes at and around 2^T and 2^30, small codes, special values, each nudged by up to two ulps.
Bounds are log-uniform over 1e-8 .. 1e2 (three of them powers of two, where s and 1/s are
exact), T is 2, 15 or 30, and every coder runs: the bitpack coder at every block size, Lorenzo
centering (both at blocks that are and are not powers of two), and the chunk coder at every
chunk size.  The encoders take these values through
their branch-free fast test, the escape shortcut for codes past 2^T, the full rule and the
neighbour retry; the whole stream (codes, widths, escapes in index order) must equal the
oracle's byte for byte, and the reconstruction must be bit-identical.
"""
import numpy as np
import pytest

import oracle
from error_bounded_lossy_encode_amd import synth
from helpers import first_difference, gpu_roundtrip, header, oracle_stream

pytestmark = pytest.mark.gpu

VARIANTS = ["bitpack", "center", "chunk4096", "chunk8192", "chunk16384"]
BLOCKS = [32, 64, 96, 128, 160, 256, 480, 512, 992, 1024, 2048]


@pytest.fixture(scope="module")
def env():
    import torch
    from error_bounded_lossy_encode_amd import binding
    binding.lib()
    return binding, torch


def case(seed: int, variant: str):
    rng = np.random.default_rng(4100 + 31 * seed + VARIANTS.index(variant))
    if seed < 3:
        eps = float(2.0 ** int(rng.integers(-26, 7)))
    else:
        eps = float(10.0 ** rng.uniform(-8, 2))
    T = [2, 15, 30][seed % 3]
    ok, eb, s, _ = oracle.resolve_bound(np.zeros(1, np.float32), False, eps)
    assert ok
    n = int(rng.integers(2, 5)) * 8192 + int(rng.integers(1, 8192))
    x = synth.adversarial(rng, n, float(eb), float(s), T)
    opts = f"abs={eps!r};outlier_log2={T}"
    if variant.startswith("chunk"):
        opts += f";coder=chunk;chunk_bytes={variant[5:]}"
    else:
        opts += f";block={int(rng.choice(BLOCKS))}"
        if variant == "center":
            opts += ";center=1"
    return x, opts


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("variant", VARIANTS)
def test_adversarial_quantizer(env, variant, seed):
    binding, torch = env
    x, opts = case(seed, variant)
    n = x.size
    print(f"[adversarial] {variant} seed {seed}: n={n} {opts}", flush=True)
    ref = oracle_stream(oracle, x, [n], opts)
    h = header(ref)
    # the stream must be coded: a raw copy would hide every quantizer decision
    assert h["mode"] in (0, 2), "adversarial field fell back to a raw copy"
    assert h["m"] > 0
    st, ref_dec = oracle.decompress(ref)
    assert st == oracle.OK
    got, dec = gpu_roundtrip(binding, torch, x, [n], opts)
    assert got.size == ref.size and np.array_equal(got, ref), f"{opts}: {first_difference(got, ref)}"
    bad = np.nonzero(dec.view(np.uint32) != ref_dec.view(np.uint32))[0]
    assert bad.size == 0, f"{opts}: reconstruction differs at {bad[:5]}"
