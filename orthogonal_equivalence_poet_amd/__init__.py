"""libpoetx: the POET-X linear layer as hand-written gfx950 HIP kernels behind a
C ABI (include/poetx.h).  ``binding`` is the ctypes layer; ``inputs`` draws the
seeded synthetic workloads; ``layer`` drives one training step of a layer."""
__all__ = ["binding", "inputs"]
