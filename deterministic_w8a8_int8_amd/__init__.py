"""Deterministic W8A8 int8 linear layer for MI355X (gfx950).

The compute path is libw8a8.so (hand-written HIP kernels behind a C ABI,
include/w8a8.h); ``binding`` is its thin ctypes binding.  ``synth`` draws
seeded synthetic inputs.  ``binding`` is imported on demand so that the
package can be imported (e.g. for ``synth``) on a machine without a GPU.
"""

__all__ = ["binding", "synth", "build"]
