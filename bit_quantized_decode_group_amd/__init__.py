"""MI355X (gfx950) 4-bit quantized decode projections.

The compute lives in ``libqgemv.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/qgemv.h``).  ``ops`` is the thin Python binding over that
ABI (argument marshalling only); ``synth`` holds the seeded synthetic input
generators.  Importing the package does not load the GPU library; the first
call into ``ops`` does, and fails loudly if it has not been built.
"""
__all__ = ["ops", "synth"]
