"""WUSH block transforms + low-bit quantization + W4A4 matmul on AMD MI355X (gfx950).

The computation lives in ``libwush.so`` (HIP kernels and a C++ host builder)
behind the C ABI declared in ``include/wush.h``; ``_lib`` is a thin ctypes
binding with the same function names, and ``layer`` adds tensor allocation
helpers around those calls.
"""

from ._lib import *  # noqa: F401,F403
from ._lib import lib, LIB_PATH, EXPORTED, WushError, FORMATS, KINDS, BLOCK  # noqa: F401
