"""Helpers for the GPU parity tests: device copies of the seeded inputs, one
full layer step through the C ABI, and error metrics."""
import numpy as np
import torch

from orthogonal_equivalence_poet_amd import binding as B

DEV = "cuda"


def tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def code(dtype: str) -> int:
    return B.POETX_BF16 if dtype == "bf16" else B.POETX_F32


def dev(a: np.ndarray, dtype: str = "f32") -> torch.Tensor:
    """Exact device copy: values are already representable in `dtype`."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(DEV).to(tdtype(dtype))


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def _rel(got, ref) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def rel_fro(got, ref) -> float:
    """Relative Frobenius error, taken over the whole tensor AND over every
    slice along the leading axis (a token row of an activation [T, d], a block
    of G / dG [nblk, b, b] or of dq [nblk, b(b-1)/2], a row of a weight), and
    the largest of these returned: a tolerance on it bounds every row or block
    on its own, so an error confined to one row, one ragged tail tile or one
    block cannot hide in the aggregate.  A slice whose reference is zero is
    measured by its absolute norm."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = _rel(got, ref)
    if got.ndim >= 2 and got.shape[0] > 1:
        g2 = got.reshape(got.shape[0], -1)
        r2 = ref.reshape(ref.shape[0], -1)
        num = np.linalg.norm(g2 - r2, axis=1)
        den = np.linalg.norm(r2, axis=1)
        err = max(err, float(np.max(num / np.where(den > 0, den, 1.0))))
    return err


def rel_fro_whole(got, ref) -> float:
    """The whole-tensor relative Frobenius error alone (for comparisons that are
    not oracle parity, e.g. a layer's output before and after a merge)."""
    return _rel(np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64))


def cnp_fwd(q: torch.Tensor, nblk: int, b: int, k: int, dtype: str) -> torch.Tensor:
    G = torch.empty((nblk, b, b), dtype=tdtype(dtype), device=DEV)
    ws = B.workspace(B.poetx_cnp_fwd_workspace_bytes(nblk, b, k, code(dtype)))
    B.poetx_cnp_fwd(q, nblk, b, k, G, ws)
    return G


def cnp_bwd(q: torch.Tensor, dG: torch.Tensor, nblk: int, b: int, k: int, dtype: str) -> torch.Tensor:
    dq = torch.empty((nblk, b * (b - 1) // 2), dtype=torch.float32, device=DEV)
    ws = B.workspace(B.poetx_cnp_bwd_workspace_bytes(nblk, b, k, code(dtype)))
    B.poetx_cnp_bwd(q, dG, nblk, b, k, dq, code(dtype), ws)
    return dq


VARIANTS = {"fast": B.POETX_FAST, "mem": B.POETX_MEM, "four_perm": B.POETX_FOUR_PERM,
            "weight_centric": B.POETX_WEIGHT_CENTRIC, "mem_q8": B.POETX_MEM_Q8}


class GpuLayer:
    """Device state of one POET-X linear plus one forward/backward step."""

    def __init__(self, spec, inp, variant=None):
        self.spec = spec
        self.variant = variant or spec.variant
        s = spec
        self.W0 = dev(inp["W0"], s.dtype)
        self.pi_R = dev_i32(inp["pi_R"])
        self.pi_P = dev_i32(inp["pi_P"])
        self.Wt = torch.empty_like(self.W0)
        B.poetx_prepermute(self.W0, self.Wt, s.m, s.n, self.pi_R, self.pi_P)
        self.q_R = dev(inp["q_R"])
        self.q_P = dev(inp["q_P"])
        self.x = dev(inp["x"], s.dtype)
        self.dy = dev(inp["dy"], s.dtype) if "dy" in inp else None
        var = VARIANTS[self.variant]
        self.desc = B.desc(s.T, s.m, s.n, s.b, s.k, code(s.dtype), var)
        # the chain variants take the pre-permuted weight, the comparison ones W0 itself,
        # the quantized one the int8 storage of the pre-permuted weight
        self.weight = self.Wt if var in (B.POETX_FAST, B.POETX_MEM) else self.W0
        if var == B.POETX_MEM_Q8:
            self.weight = B.workspace(B.poetx_qweight_bytes(s.m, s.n))
            B.poetx_quantize_weight(self.Wt, s.m, s.n, self.weight)

    def forward(self):
        s = self.spec
        self.G_R = cnp_fwd(self.q_R, s.nblk_R, s.b, s.k, s.dtype)
        self.G_P = cnp_fwd(self.q_P, s.nblk_P, s.b, s.k, s.dtype)
        self.y = torch.empty((s.T, s.m), dtype=tdtype(s.dtype), device=DEV)
        nsaved = B.poetx_linear_saved_bytes(self.desc)
        self.saved = B.workspace(nsaved)
        ws = B.workspace(B.poetx_linear_fwd_workspace_bytes(self.desc))
        B.poetx_linear_fwd(self.desc, self.x, self.weight, self.G_R, self.G_P, self.pi_R, self.pi_P, self.y,
                           self.saved, ws)
        return self.y

    def backward(self):
        s = self.spec
        self.dx = torch.empty((s.T, s.n), dtype=tdtype(s.dtype), device=DEV)
        self.dG_R = torch.empty((s.nblk_R, s.b, s.b), dtype=torch.float32, device=DEV)
        self.dG_P = torch.empty((s.nblk_P, s.b, s.b), dtype=torch.float32, device=DEV)
        ws = B.workspace(B.poetx_linear_bwd_workspace_bytes(self.desc))
        B.poetx_linear_bwd(self.desc, self.dy, self.x, self.weight, self.G_R, self.G_P, self.pi_R, self.pi_P,
                           self.saved, self.dx, self.dG_R, self.dG_P, ws)
        self.dq_R = cnp_bwd(self.q_R, self.dG_R, s.nblk_R, s.b, s.k, s.dtype)
        self.dq_P = cnp_bwd(self.q_P, self.dG_P, s.nblk_P, s.b, s.k, s.dtype)
        return self.dx


def tol(dtype: str) -> float:
    """Relative Frobenius bound: 1e-5 on the float32 path, 1.5e-2 for bf16
    operands with float32 accumulation."""
    return 1e-5 if dtype == "f32" else 1.5e-2
