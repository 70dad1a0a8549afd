"""MI355X-native constant-shape transformer decode step.

The hot path lives in libds3.so (HIP kernels for gfx950 behind the C ABI of include/ds3.h); this package is its
build script and a thin ctypes binding. There is no CPU fallback: without the built library every entry point
raises.
"""
from . import _ds3
from ._ds3 import DS3Error, load_library  # noqa: F401
from .engine import Engine, make_config  # noqa: F401

__all__ = ["Engine", "make_config", "DS3Error", "load_library", "_ds3"]
