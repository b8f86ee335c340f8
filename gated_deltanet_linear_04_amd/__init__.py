"""MI355X (gfx950) gated delta rule prefill: HIP kernels behind a C ABI.

The native library ``libgdn.so`` (built from ``csrc/``) exports the calls
declared in ``include/gdn.h``; ``gated_deltanet_linear_04_amd.binding`` is a
thin ctypes layer over it that marshals torch tensors into plain device
pointers.  ``synth`` holds the seeded input generators.
"""
from __future__ import annotations

__all__ = ["binding", "synth"]


def __getattr__(name):
    # Lazy: importing the package must not require the built library (the
    # CPU-only tests import ``synth``).  Accessing ``binding`` loads it and
    # fails loudly if it is missing.
    if name == "binding":
        from . import binding
        return binding
    raise AttributeError(name)
