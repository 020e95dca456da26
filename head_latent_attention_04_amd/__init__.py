"""Weight-absorbed MLA decode and chunked prefill on MI355X (gfx950).

The computation lives in libmla.so (hand-written HIP kernels behind the C ABI of
include/mla.h); `lib` is its thin ctypes binding.
"""
from . import lib  # noqa: F401
