"""MI355X-native error-bounded lossy compressor for float32 fields.

The codec runs in hand-written HIP kernels for gfx950 inside ``libeblc.so`` (C ABI declared in
``include/eblc.h``).  ``binding`` wraps that ABI with ctypes under the same names; it loads the
library on first use and raises if it is missing.  ``synth`` makes the seeded synthetic inputs.
"""
__all__ = ["binding", "synth"]
