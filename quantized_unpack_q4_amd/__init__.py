"""Fused Q8_0 / Q4_K block-dequant matmul for AMD MI355X (gfx950).

The compute lives in ``libgq.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/gq.h``); :mod:`quantized_unpack_q4_amd.gq` is the thin
ctypes binding with the same entry-point names.  Importing this package does
not load the library; the first call through the binding does, and fails
loudly if it has not been built.
"""
__version__ = "0.1.0"
