"""MI355X-native DFlash + DDTree draft-and-verify kernel chain.

The compute lives in ``libddt.so`` (hand-written HIP kernels for gfx950 behind
the C ABI in ``include/ddt.h``); ``ddt`` is its thin Python binding.
"""
from . import ddt  # noqa: F401

__all__ = ["ddt"]
