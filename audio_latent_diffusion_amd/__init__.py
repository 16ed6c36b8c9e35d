"""MI355X (gfx950) DiT denoise step for text-conditioned audio latent diffusion.

The computation lives in libald.so (hand-written HIP kernels behind the C ABI
declared in include/ald.h).  This package holds the ctypes declarations
(_lib), a thin binding with one Python function per C entry point (binding),
and the device-resident model / step runner (runtime).  Importing the package
does not load the library; the first call does, and fails loudly if it has
not been built.
"""
from . import _lib  # noqa: F401

__all__ = ["_lib", "binding", "runtime"]
