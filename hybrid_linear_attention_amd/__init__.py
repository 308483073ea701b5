"""Gated DeltaNet recurrence on AMD MI355X (gfx950).

The C-ABI library ``libgdn.so`` (declared in ``include/gdn.h``) holds the HIP
kernels; ``hybrid_linear_attention_amd.gdn`` is its Python binding.  The
binding is imported on first attribute access so that importing the package
alone (for the build step) does not require the built library.
"""
import importlib

__all__ = ["gdn", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
