"""MI355X (gfx950) Spark-Attn block-sparse video attention layer.

The layer's five stages run in the HIP kernels of libbsattn.so, reached through the C ABI in
include/bsattn.h; `ops` re-exports the thin torch-facing binding.  Importing the package does
not load the library; the first call does, and fails loudly if it has not been built.
"""
from . import synth  # noqa: F401


def __getattr__(name):
    if name == "ops":
        from . import _lib
        return _lib
    raise AttributeError(name)
