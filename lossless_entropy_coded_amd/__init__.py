"""lossless_entropy_coded_amd -- lossless entropy-coded bf16 weights for MI355X.

bf16 weights are split into an 8-bit exponent, Huffman-coded, and a raw
sign+mantissa byte; a gfx950 HIP kernel decodes a whole container back into
bit-identical bf16 in one launch.  The native library is reached through
``lossless_entropy_coded_amd.wc`` (ctypes binding of include/wc.h); the
seeded workload generators live in ``lossless_entropy_coded_amd.synth``.
"""
__all__ = ["wc", "synth"]
