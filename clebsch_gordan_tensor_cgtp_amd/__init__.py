"""MI355X-native fused Clebsch-Gordan tensor-product convolution.

The compute lives in ``libcgtp.so`` (C ABI, HIP kernels for gfx950); the
Python side is a thin ctypes binding (``binding``) plus seeded input
generators (``synth``).  Importing the package does not load the library;
the first call into ``binding`` does, and fails loudly if it is missing.
"""
__all__ = ["binding", "synth"]
