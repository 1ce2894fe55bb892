"""VC-Attention (V-Smooth + ExpCast-FP8) for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library libvcattn.so (C ABI:
include/vc_attention.h); ``_lib`` is its ctypes binding under the C names and
``api`` adds torch-tensor conveniences (output allocation only).  ``synth``
draws the seeded synthetic inputs.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "api"]


def __getattr__(name):
    if name in ("api", "_lib"):
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
