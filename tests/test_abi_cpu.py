"""CPU checks of the library boundary: it loads, exports every declared symbol, and answers the
calls that need no GPU."""
import ctypes
import os
import re

import pytest

from error_bounded_lossy_encode_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "eblc.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(eblc_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = binding.lib()
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(binding.EXPORTS)


def test_calls_without_gpu():
    assert binding.eblc_abi_version() == 1
    assert binding.eblc_status_string(binding.EBLC_CORRUPT_STREAM) == "corrupt stream"
    assert binding.eblc_status_string(99) == "unknown status"
    lib = binding.lib()
    assert lib.eblc_max_compressed_bytes(None) == 0
    assert lib.eblc_payload_alignment(None) == 0
    assert lib.eblc_plan_limits(None, None) == binding.EBLC_INVALID_ARGUMENT
    assert lib.eblc_compress_batch(None, 0, None, None, None, None, None) == binding.EBLC_INVALID_ARGUMENT
    assert lib.eblc_decompress_batch(None, 0, None, None, None, None) == binding.EBLC_INVALID_ARGUMENT
    assert lib.eblc_plan_set_profiling(None, 4, None, 1) == binding.EBLC_INVALID_ARGUMENT
    assert lib.eblc_plan_kernel_times(None, None, None, None, 0) == -1
    lib.eblc_plan_destroy(None)


@pytest.mark.parametrize("kind", [binding.EBLC_EXECUTION_HOST, binding.EBLC_EXECUTION_CUDA])
def test_unsupported_execution_kinds(kind):
    st, plan = binding.eblc_plan_create([64, 64], "rel=1e-3", kind=kind)
    assert st == binding.EBLC_UNSUPPORTED and plan is None


@pytest.mark.parametrize("opts", ["rel=-1", "abs=nan", "rel=1e-3;abs=1", "block=48", "block=4096",
                                  "block=0", "block=16", "block=1056", "block=1536", "block=2016",
                                  "outlier_log2=0", "outlier_log2=31", "bogus=1", "rel", "side_max=-3",
                                  "block=256;block=128", "side_max=5000", "coder=huffman",
                                  "coder=chunk;block=256", "chunk_bytes=8192", "coder=chunk;chunk_bytes=2048",
                                  "coder=chunk;chunk_bytes=32768", "coder=chunk;coder=chunk",
                                  "coder=chunk;chunk_bytes=4096;chunk_bytes=4096",
                                  "center=2", "center=1;center=1", "center=yes", "coder=chunk;center=1",
                                  "lanes=0", "lanes=9", "lanes=-1", "lanes=2;lanes=2", "lanes=two"])
def test_invalid_options_rejected_before_any_device_call(opts):
    st, plan = binding.eblc_plan_create([64, 64], opts)
    assert st == binding.EBLC_INVALID_ARGUMENT and plan is None


def test_shape_checks():
    assert binding.eblc_plan_create([64, 0])[0] == binding.EBLC_INVALID_ARGUMENT
    assert binding.eblc_plan_create([1] * 5)[0] == binding.EBLC_UNSUPPORTED
    assert binding.eblc_plan_create([1 << 16, 1 << 16])[0] == binding.EBLC_INVALID_ARGUMENT
    # row-major with padding is a supported layout; these are not: fastest stride other than 1
    # (transposed), overlapping rows, zero or negative strides
    for dims, strides in (([8, 8], [1, 8]), ([8, 8], [4, 1]), ([8, 8], [16, 2]), ([8, 8], [0, 1]),
                          ([4, 4, 4], [16, -4, 1]), ([4, 4, 4], [8, 4, 1])):
        assert binding.eblc_plan_create(dims, strides=strides)[0] == binding.EBLC_UNSUPPORTED, strides
    assert binding.eblc_plan_create([8, 8], dtype=3)[0] == binding.EBLC_UNSUPPORTED


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.parametrize("block", [32, 96, 160, 480, 992, 1024, 2048])
def test_block_grammar_accepts_multiples_of_32(block):
    """Every multiple of 32 up to 1024, and 2048, passes the option checks: without a GPU the
    plan then stops at the device query."""
    if _gpu_visible():
        pytest.skip("checks the option parser on a host without a GPU")
    st, plan = binding.eblc_plan_create([4096], f"rel=1e-3;block={block}")
    assert st == binding.EBLC_DEVICE_ERROR and plan is None


def test_payload_word_limit():
    """The scans count payload words in 32 bits, so a plan is refused when its field's largest
    payload reaches 2^32 words: 32 words per 32-value segment for the bitpack coder (n above
    2^32 - 32), the bitmap and every plane word of every chunk for the chunk coder."""
    if _gpu_visible():
        pytest.skip("checks the plan limits on a host without a GPU")
    lim_bitpack = (1 << 32) - 32
    assert binding.eblc_plan_create([lim_bitpack + 1], "rel=1e-3")[0] == binding.EBLC_INVALID_ARGUMENT
    assert binding.eblc_plan_create([lim_bitpack], "rel=1e-3")[0] == binding.EBLC_DEVICE_ERROR
    for chunk_bytes in (4096, 8192, 16384):
        V = chunk_bytes // 4
        chunks = ((1 << 32) - 1) // (V + V // 32)     # the most chunks below the limit
        opts = f"rel=1e-3;coder=chunk;chunk_bytes={chunk_bytes}"
        n_ok = min(chunks * V, (1 << 32) - 1)
        assert binding.eblc_plan_create([n_ok], opts)[0] == binding.EBLC_DEVICE_ERROR, chunk_bytes
        if n_ok < (1 << 32) - 1:
            assert binding.eblc_plan_create([n_ok + 1], opts)[0] == binding.EBLC_INVALID_ARGUMENT, chunk_bytes


@pytest.mark.parametrize("opts", ["rel=1e-3;block=32;center=1", "rel=1e-3;block=96;center=1",
                                  "rel=1e-3;coder=chunk;chunk_bytes=4096", "rel=1e-3;coder=chunk;chunk_bytes=16384",
                                  "abs=1e-3;block=2048"])
def test_noalloc_scratch_limit(opts):
    """eblc_compress_noalloc checks the field against its static scratch before any device call:
    every coder and option fits at 2^22 values (the call then stops at the device query), one
    more value is refused."""
    if _gpu_visible():
        pytest.skip("checks the size limit on a host without a GPU")
    lib = binding.lib()
    ex = binding.eblc_execution_t(binding.EBLC_EXECUTION_HIP, 0, 0)
    res = ctypes.create_string_buffer(32)
    addr = (ctypes.addressof(res) + 15) // 16 * 16
    for n, want in (((1 << 22), binding.EBLC_DEVICE_ERROR), ((1 << 22) + 1, binding.EBLC_TOO_LARGE)):
        d = (ctypes.c_int64 * 1)(n)
        st = lib.eblc_compress_noalloc(ctypes.byref(ex), 1, d, None, opts.encode(), None, None, 0,
                                       ctypes.c_void_p(addr), None)
        assert st == want, (n, st)
