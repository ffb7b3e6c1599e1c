"""BitNet b1.58 BitLinear forward pass on AMD Instinct MI355X (gfx950).

The compute lives in ``csrc/`` (hand-written HIP kernels behind a C ABI,
declared in ``include/bitlinear.h``) and is built into ``libbitlinear.so``.
``bitlinear`` is the thin ctypes binding with the same call names; it fails
loudly when the built library is missing.  ``synthetic`` holds the seeded
input generators.
"""
__all__ = ["bitlinear", "synthetic"]
