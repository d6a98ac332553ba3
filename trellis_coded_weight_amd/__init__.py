"""MI355X (gfx950) bitshift-trellis quantisation kernels: batched Viterbi encoding with
computed codes (1MAD, 3INST), parallel window decode and BCJR soft relaxation.

The product is the C ABI in ``include/qtcq.h`` (``libqtcq.so``); ``_native`` binds it
with ctypes and ``api`` adds torch allocation helpers.  Submodules load lazily so that
``inputs`` (seeded synthetic data) can be imported without the native library.
"""
import importlib

__all__ = ["api", "inputs", "build"]


def __getattr__(name):
    if name in ("api", "inputs", "build", "_native"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
