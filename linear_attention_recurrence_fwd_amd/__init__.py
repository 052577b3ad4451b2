"""Gated delta rule (GatedDeltaNet) forward scan and VJP on MI355X (gfx950).

The compute lives in ``libgdn.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/gdn.h``); ``binding`` marshals torch tensors to it.
``inputs`` holds the seeded synthetic workloads.  The binding is imported
lazily so that ``inputs`` works on machines without the built library.
"""
import importlib

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(__name__ + "." + name)
    raise AttributeError(name)
