"""Seeded synthetic inputs for the POET-X linear layer.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the layer's arithmetic, so the oracle and the HIP path can
both be fed from it without sharing any computation.

Recipe (every workload):
  * one ``numpy.random.default_rng`` stream per tensor, keyed by
    ``(workload_id, layer_id, linear_id, tensor_id)``;
  * tensor ids: 0 W0, 1 q_R, 2 q_P, 3 x, 4 pi_R, 5 pi_P, 6 dY, 7 pi_R', 8 pi_P';
  * Gaussian values are drawn in float64, scaled by their standard deviation,
    rounded to float32 and then (for bf16 workloads) to bf16 with
    round-to-nearest-even, so every array returned here is exactly
    representable in the dtype the GPU receives;
  * permutations are ``rng.permutation(d)`` as int32; the upper-triangle
    parameters are always float32.

The shapes follow Llama-8B / Llama-13B linears (the pages' pretraining models);
the text corpus the pages train on is not needed and not used: Gaussian
activations of the same shapes stand in for it.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

W0_ID, QR_ID, QP_ID, X_ID, PIR_ID, PIP_ID, DY_ID, PIR2_ID, PIP2_ID = range(9)


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    Finite inputs only (the generators never produce NaN or Inf).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32)


def gaussian(shape, std: float, dtype: str, *key: int) -> np.ndarray:
    g = rng(*key)
    v = (g.standard_normal(size=shape) * std).astype(np.float32)
    if dtype == "bf16":
        v = round_to_bf16(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return v


def permutation(d: int, *key: int) -> np.ndarray:
    return rng(*key).permutation(d).astype(np.int32)


@dataclass
class LinearSpec:
    """One POET-X linear: W0 is m x n (d_out x d_in), block size b on both sides."""
    name: str
    m: int
    n: int
    b: int
    k: int
    T: int
    dtype: str                 # "f32" or "bf16": activations, W0 and the G blocks
    w_std: float = 0.02
    q_std: float = 1e-3
    x_std: float = 1.0
    variant: str = "fast"      # "fast" or "mem"
    q_block_norm: Optional[float] = None   # target spectral norm of every Q block
    key: tuple = (0, 0, 0)     # (workload_id, layer_id, linear_id)

    @property
    def nblk_R(self) -> int:
        return self.m // self.b

    @property
    def nblk_P(self) -> int:
        return self.n // self.b

    @property
    def ntri(self) -> int:
        return self.b * (self.b - 1) // 2


def make_linear_inputs(spec: LinearSpec, with_grad: bool = True,
                       with_new_perm: bool = False) -> Dict[str, np.ndarray]:
    """Draw every input of one linear. q_R / q_P are *not* rescaled here even
    when ``q_block_norm`` is set (that needs the skew layout; callers do it)."""
    k0 = spec.key
    out = {
        "W0": gaussian((spec.m, spec.n), spec.w_std, spec.dtype, *k0, W0_ID),
        "q_R": gaussian((spec.nblk_R, spec.ntri), spec.q_std, "f32", *k0, QR_ID),
        "q_P": gaussian((spec.nblk_P, spec.ntri), spec.q_std, "f32", *k0, QP_ID),
        "x": gaussian((spec.T, spec.n), spec.x_std, spec.dtype, *k0, X_ID),
        "pi_R": permutation(spec.m, *k0, PIR_ID),
        "pi_P": permutation(spec.n, *k0, PIP_ID),
    }
    if with_grad:
        out["dy"] = gaussian((spec.T, spec.m), 1.0, spec.dtype, *k0, DY_ID)
    if with_new_perm:
        out["pi_R_new"] = permutation(spec.m, *k0, PIR2_ID)
        out["pi_P_new"] = permutation(spec.n, *k0, PIP2_ID)
    return out


# ----------------------------------------------------------------- workloads
def tiny() -> LinearSpec:
    """Tiny fp32 linear: 64 x 64, b=16 (4 blocks per side), k=3, 32 tokens."""
    return LinearSpec("tiny_64x64_b16", m=64, n=64, b=16, k=3, T=32, dtype="f32",
                      w_std=0.02, q_std=0.05, key=(1, 0, 0))


def llama8b_q_proj() -> LinearSpec:
    """Llama-8B q_proj: 4096 x 4096, b=256, k=3, 1 x 2048 tokens, bf16, fast."""
    return LinearSpec("llama8b_q_proj", m=4096, n=4096, b=256, k=3, T=2048,
                      dtype="bf16", w_std=0.02, q_std=1e-3, variant="fast",
                      key=(2, 0, 0))


def llama8b_up_proj(variant: str = "fast") -> LinearSpec:
    """Llama-8B MLP up_proj: 14336 x 4096, b=512, k=4, 2 x 2048 tokens, bf16,
    q ~ N(0, 1e-2^2) rescaled so that every Q block has spectral norm 0.5."""
    return LinearSpec("llama8b_up_proj", m=14336, n=4096, b=512, k=4, T=4096,
                      dtype="bf16", w_std=0.02, q_std=1e-2, variant=variant,
                      q_block_norm=0.5, key=(3, 0, 0))


_LLAMA8B_SHAPES = [  # (name, d_out, d_in): hidden 4096, 32 q / 8 kv heads of 128, FFN 14336
    ("q_proj", 4096, 4096), ("k_proj", 1024, 4096), ("v_proj", 1024, 4096),
    ("o_proj", 4096, 4096), ("gate_proj", 14336, 4096), ("up_proj", 14336, 4096),
    ("down_proj", 4096, 14336)]

_LLAMA13B_SHAPES = [  # hidden 5120, 40 heads of 128, FFN 13824
    ("q_proj", 5120, 5120), ("k_proj", 5120, 5120), ("v_proj", 5120, 5120),
    ("o_proj", 5120, 5120), ("gate_proj", 13824, 5120), ("up_proj", 13824, 5120),
    ("down_proj", 5120, 13824)]


def llama8b_layer() -> List[LinearSpec]:
    """All 7 linears of one Llama-8B decoder layer, mem variant, b=256, k=3, 2048 tokens."""
    return [LinearSpec(f"llama8b_{nm}", m=mo, n=ni, b=256, k=3, T=2048, dtype="bf16",
                       variant="mem", key=(4, 0, i))
            for i, (nm, mo, ni) in enumerate(_LLAMA8B_SHAPES)]


def llama13b_layer() -> List[LinearSpec]:
    """All 7 linears of one Llama-13B decoder layer, mem variant, b=256, k=3, 4 x 2048 tokens."""
    return [LinearSpec(f"llama13b_{nm}", m=mo, n=ni, b=256, k=3, T=8192, dtype="bf16",
                       variant="mem", key=(5, 0, i))
            for i, (nm, mo, ni) in enumerate(_LLAMA13B_SHAPES)]


def llama13b_cnp_blocks(layers: int = 40, b: int = 256) -> int:
    """Number of b x b blocks of every POET-X linear in ``layers`` Llama-13B layers."""
    return layers * sum(mo // b + ni // b for _, mo, ni in _LLAMA13B_SHAPES)


def cnp_params(nblk: int, b: int, std: float, *key: int) -> np.ndarray:
    """Upper-triangle parameters for a flat batch of blocks (float32)."""
    return gaussian((nblk, b * (b - 1) // 2), std, "f32", *key)
