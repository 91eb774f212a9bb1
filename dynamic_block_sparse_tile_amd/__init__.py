"""Dynamic tile-sparse global (cross-frame) attention for MI355X (gfx950).

The compute lives in ``libsparse3d.so`` (hand-written HIP kernels behind the C ABI
in ``include/sparse3d.h``); ``sparse3d`` is its ctypes binding, ``layer`` composes
one layer from the calls, ``synth`` draws seeded multi-view inputs.  Submodules are
imported on first use so that ``synth`` works without the built library.
"""
import importlib

__all__ = ["sparse3d", "layer", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
