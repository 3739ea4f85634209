"""MI355X (gfx950) streaming chunk attention: 3D RoPE at a global time index,
a sink-pinned ring KV cache and block-causal chunk attention, as hand-written
HIP kernels behind a C ABI (``include/scv.h``, ``libscv.so``).

The Python side is argument marshalling only (``binding``); every step of the
path runs in the library's kernels.
"""

__all__ = ["binding", "workloads", "datagen"]
