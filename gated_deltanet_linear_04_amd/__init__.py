"""MI355X (gfx950) gated delta rule prefill: HIP kernels behind a C ABI.

The native library ``libgdn.so`` (built from ``csrc/`` by ``build.py``)
exports the calls declared in ``include/gdn.h``; ``binding`` is a thin ctypes
layer over it that marshals torch tensors into plain device pointers and
loads the library on first use (failing loudly if it is not built).
``synth`` holds the seeded input generators.
"""
