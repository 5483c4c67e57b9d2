"""Whisper large-v3 inference hot path on MI355X (gfx950).

The computation lives in libwhisper_mi355x.so (hand-written HIP kernels
behind the C ABI in include/whisper_mi355x.h). `_lib` is the ctypes binding
with the ABI's names; `runtime` allocates device buffers with torch and
passes pointers.
"""
from . import _lib  # noqa: F401
from ._lib import LIB_PATH, WhisperError, make_dims  # noqa: F401
