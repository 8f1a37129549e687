"""MI355X-native forward pass of 2D (dilated) Neighborhood Attention.

The compute lives in ``libna2d.so`` (hand-written HIP kernels for gfx950 behind
a C ABI declared in ``include/na2d.h``); ``vision_transformer_local_amd.na2d``
is the thin ctypes binding.  Importing this package loads nothing; the
library is loaded on first use and a missing library is a hard error.
"""
__all__ = ["na2d", "inputs"]
