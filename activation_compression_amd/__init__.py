"""COAT-style FP8 compression of AdamW optimizer states and activations,
native to one AMD MI355X (gfx950).

The path runs in hand-written HIP kernels behind the C ABI declared in
``include/coat.h`` (``libcoat.so``, built by ``build.py``); ``coat`` is its
thin Python binding and ``inputs`` draws the seeded synthetic workloads.
Importing the package loads nothing; the library is loaded on first use.
"""
