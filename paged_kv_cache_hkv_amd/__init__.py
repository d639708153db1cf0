"""Paged KV-cache attention for one mixed continuous batch on AMD MI355X (gfx950).

The compute path is ``libpa.so`` (hand-written HIP kernels behind the C ABI of
``include/pa.h``); ``binding`` marshals torch tensors into it and ``synth``
draws seeded synthetic inputs.  ``build`` compiles the library in-tree.
"""

__all__ = ["binding", "synth", "build"]
