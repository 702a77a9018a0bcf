"""MI355X-native FLUX-style MMDiT denoising step.

The compute runs in hand-written HIP kernels for gfx950 inside
``libmmdit.so`` (C ABI declared in ``include/mmdit.h``). ``binding`` is a thin
ctypes layer over it; ``inputs`` draws seeded synthetic inputs and weights.
Importing this package does not load the library; ``binding.lib()`` does,
and raises if it has not been built.
"""
__all__ = ["binding", "inputs"]
