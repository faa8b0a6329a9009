"""MI355X-native compressed-attention decode (DeepSeek-V4 CSA / HCA) for one layer.

The compute lives in ``libcsa.so`` (hand-written HIP for gfx950, C ABI declared
in ``include/csa.h``).  ``_lib`` is the ctypes binding with the same function
names; ``synth`` holds the seeded synthetic workloads.  The library is loaded
on first use and its absence is an error.
"""

from . import _lib  # noqa: F401
from ._lib import (BF16, F32, FP4_E4M3_16, FP8_MX32, WIN_LINEAR, WIN_RING128,  # noqa: F401
                   CsaError, lib)
