"""MI355X-native lightning-indexer sparse-attention decode step.

The compute lives in ``liblsi.so`` (hand-written HIP for gfx950 behind a
C ABI, declared in ``include/lsi.h``).  This package holds the thin ctypes
binding (``lsi``), the seeded input generators (``synth``) and the build
helper (``build``).  Importing the package does not load the library; the
first call through the binding does, and it raises if the library is absent.
"""
__all__ = ["lsi", "synth", "build"]
