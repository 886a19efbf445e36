"""libpoetx: the POET-X linear layer as hand-written gfx950 HIP kernels behind a
C ABI (include/poetx.h).  ``binding`` is the ctypes layer; ``layer`` wraps one
linear as a torch module (POETLinear: autograd forward and backward, the
library's AdamW step and merge-then-reinitialize); ``inputs`` draws the seeded
synthetic workloads."""
__all__ = ["binding", "inputs", "layer"]
