"""MXFP4 W4A8 linear layer for MI355X (gfx950): Python binding of libw4a8.so.

The binding only marshals arguments (torch tensors -> device pointers, the
current HIP stream) and maps status codes to exceptions; every step of the
computation runs in the library's HIP kernels.  The library is loaded on the
first call and its absence is an error: there is no fallback path.
"""
from .binding import *  # noqa: F401,F403
from .binding import __all__  # noqa: F401
