"""NABLA (Neighborhood Adaptive Block-Level Attention) on AMD MI355X (gfx950).

The computation lives in libnabla.so (hand-written HIP kernels behind the C ABI
of include/nabla.h); this package is its thin Python binding.
"""
from .api import *  # noqa: F401,F403
from .api import __all__  # noqa: F401
