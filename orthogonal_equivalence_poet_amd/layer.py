"""POETLinear: one POET-X linear as a torch module.

The layer trains a frozen weight W0 through y = R W0 P x ("POET-X: Memory-efficient
LLM Training by Scaling Orthogonal Transformation", SAI replication review,
Summary; the agidaily.cc article): R and P are block-diagonal orthogonal
transforms in random permuted bases, every block a Cayley-Neumann series of a
skew-symmetric Q kept as its upper triangle (the trainable parameters q_R, q_P).
The review's Summary names the pieces this module exposes: the fast and the
checkpointed mem variant (``mem_efficient_mode``), the quantized variant on top
of it (``quantized``: POET-XQ, the weight kept as int8 per output row and
expanded inside each library call) and merge-then-reinitialize
(``merge_then_reinitialize``).

Everything the layer computes runs in libpoetx (``binding``): this module only
owns the device buffers (the pre-permuted weight, the permutations, the
parameters and the optimizer moments) and orders the library calls.  Forward and
backward go through ``torch.autograd``; ``optimizer_step`` is the library's
AdamW at the POET-scaled rate, and a merge resets its moments and count.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return B.POETX_BF16
    if dtype == torch.float32:
        return B.POETX_F32
    raise TypeError(f"unsupported dtype {dtype}")


def _perm(d: int, generator: Optional[torch.Generator], device) -> torch.Tensor:
    return torch.randperm(d, generator=generator).to(device=device, dtype=torch.int32)


class _CayleyNeumannFn(torch.autograd.Function):
    """G = (I + Q) sum_{i<=k} Q^i for every block of q [nblk, b(b-1)/2]."""

    @staticmethod
    def forward(ctx, q, b, k, dtype):
        nblk = q.shape[0]
        code = _code(dtype)
        q = q.detach().contiguous()
        G = torch.empty((nblk, b, b), dtype=dtype, device=q.device)
        ws = B.workspace(B.poetx_cnp_fwd_workspace_bytes(nblk, b, k, code), q.device)
        saved = B.workspace(B.poetx_cnp_saved_bytes(nblk, b, k, code), q.device)
        B.poetx_cnp_fwd_save(q, nblk, b, k, G, saved, ws)
        ctx.stash = (q, b, k, code, saved)
        return G

    @staticmethod
    def backward(ctx, dG):
        q, b, k, code, saved = ctx.stash
        ctx.stash = None
        dq = torch.empty_like(q)
        ws = B.workspace(B.poetx_cnp_bwd_workspace_bytes(q.shape[0], b, k, code), q.device)
        B.poetx_cnp_bwd_saved(q, dG.float().contiguous(), q.shape[0], b, k, dq, code, saved, ws)
        return dq, None, None, None


def cayley_neumann(q: torch.Tensor, b: int, k: int = 3, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """The orthogonal blocks of the compact parameters q [nblk, b(b-1)/2] (float32,
    on a GPU): G [nblk, b, b] in `dtype`, differentiable with respect to q.  The
    review's Summary names the fused Cayley-Neumann transform as a separate
    operator; this is that operator over any number of blocks."""
    return _CayleyNeumannFn.apply(q, int(b), int(k), dtype)


class _PoetLinearFn(torch.autograd.Function):
    """y = R W0 P x for x [T, n]; gradients for x, q_R and q_P (none for W0).

    What lives from the forward to the backward is exactly what the variant
    saves (the review's Summary and Reproducibility & code: POET-X_fast keeps
    intermediates, the checkpointed POET-X_mem recomputes them):
      fast: the blocks G, the transform's saved Q / Q^2 terms and the chain's
            saved h2 and gathered input (poetx_linear_saved_bytes);
      mem (and the quantized layer): nothing beyond x and the parameters; the
            backward forms G again from q.
    Workspaces are taken inside each call and released before it returns."""

    @staticmethod
    def forward(ctx, x, q_R, q_P, layer):
        T = x.shape[0]
        d = layer._desc(T)
        nR, nblk, b, k = layer.nblk_R, layer.nblk, layer.block_size, layer.k
        code = _code(layer.dtype)
        q = torch.cat([q_R.detach(), q_P.detach()]).contiguous()   # one flat batch of blocks
        G = torch.empty((nblk, b, b), dtype=layer.dtype, device=x.device)
        y = torch.empty((T, layer.out_features), dtype=x.dtype, device=x.device)
        ws = B.workspace(max(B.poetx_linear_fwd_workspace_bytes(d),
                             B.poetx_cnp_fwd_workspace_bytes(nblk, b, k, code)), x.device)
        if layer.mem_efficient_mode:
            B.poetx_cnp_fwd(q, nblk, b, k, G, ws)
            B.poetx_linear_fwd(d, x, layer.weight, G[:nR], G[nR:], layer.pi_R, layer.pi_P, y, None, ws)
            ctx.stash = (layer, d, None, None, None)
        else:
            cnp_saved = B.workspace(B.poetx_cnp_saved_bytes(nblk, b, k, code), x.device)
            saved = B.workspace(B.poetx_linear_saved_bytes(d), x.device)
            B.poetx_cnp_fwd_save(q, nblk, b, k, G, cnp_saved, ws)
            B.poetx_linear_fwd(d, x, layer.weight, G[:nR], G[nR:], layer.pi_R, layer.pi_P, y, saved, ws)
            ctx.stash = (layer, d, G, cnp_saved, saved)
        ctx.save_for_backward(x, q_R, q_P)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, q_R, q_P = ctx.saved_tensors
        layer, d, G, cnp_saved, saved = ctx.stash
        ctx.stash = None
        nR, nblk, b, k = layer.nblk_R, layer.nblk, layer.block_size, layer.k
        code = _code(layer.dtype)
        q = torch.cat([q_R.detach(), q_P.detach()]).contiguous()
        dy = dy.to(x.dtype).contiguous()
        dx = torch.empty_like(x)
        dG = torch.empty((nblk, b, b), dtype=torch.float32, device=x.device)
        dq = torch.empty_like(q)
        ws = B.workspace(max(B.poetx_linear_bwd_workspace_bytes(d),
                             B.poetx_cnp_fwd_workspace_bytes(nblk, b, k, code),
                             B.poetx_cnp_bwd_workspace_bytes(nblk, b, k, code)), x.device)
        if G is None:
            # mem: the blocks again from q, keeping the transform's terms for its backward
            G = torch.empty((nblk, b, b), dtype=layer.dtype, device=x.device)
            cnp_saved = B.workspace(B.poetx_cnp_saved_bytes(nblk, b, k, code), x.device)
            B.poetx_cnp_fwd_save(q, nblk, b, k, G, cnp_saved, ws)
        B.poetx_linear_bwd(d, dy, x, layer.weight, G[:nR], G[nR:], layer.pi_R, layer.pi_P, saved, dx, dG[:nR],
                           dG[nR:], ws)
        B.poetx_cnp_bwd_saved(q, dG, nblk, b, k, dq, code, cnp_saved, ws)
        return dx, dq[:nR], dq[nR:], None


class POETLinear(torch.nn.Module):
    """A linear layer trained as y = R W0 P x with W0 frozen.

    W0: [out_features, in_features] float32 or bfloat16 on a GPU; its dtype is the
    layer's compute dtype (activations must match).  block_size must divide both
    feature counts and be a multiple of 16; k is the Neumann order.  q_R and q_P
    start at zero (R = P = I), so the layer starts as x W0^T.  quantized=True
    (bfloat16 only, implies the mem variant) keeps the pre-permuted weight as
    int8 codes with one scale per output row instead of the weight itself.
    """

    def __init__(self, W0: torch.Tensor, block_size: int, k: int = 3, mem_efficient_mode: bool = False,
                 generator: Optional[torch.Generator] = None, quantized: bool = False):
        super().__init__()
        B.load()
        m, n = W0.shape
        b = int(block_size)
        if m % b or n % b:
            raise ValueError(f"block size {b} must divide both {m} and {n}")
        self.out_features, self.in_features, self.block_size, self.k = m, n, b, int(k)
        self.quantized = bool(quantized)
        if self.quantized and W0.dtype != torch.bfloat16:
            raise TypeError("the quantized layer computes in bfloat16")
        if self.quantized and b % 64:
            raise ValueError("the quantized layer needs a block size that is a multiple of 64")
        self.mem_efficient_mode = bool(mem_efficient_mode) or self.quantized
        self.dtype = W0.dtype
        self.nblk_R, self.nblk_P = m // b, n // b
        self.nblk = self.nblk_R + self.nblk_P
        ntri = b * (b - 1) // 2
        dev = W0.device
        self.register_buffer("pi_R", _perm(m, generator, dev))
        self.register_buffer("pi_P", _perm(n, generator, dev))
        W0 = W0.detach().contiguous()
        Wt = torch.empty_like(W0)
        B.poetx_prepermute(W0, Wt, m, n, self.pi_R, self.pi_P)
        if self.quantized:
            # int8 codes [m, n] then float32 row scales, one byte buffer (the library's layout)
            self.register_buffer("Wq", B.workspace(B.poetx_qweight_bytes(m, n), dev))
            B.poetx_quantize_weight(Wt, m, n, self.Wq)
            del Wt
        else:
            self.register_buffer("Wt", Wt)
        self.q_R = torch.nn.Parameter(torch.zeros((self.nblk_R, ntri), dtype=torch.float32, device=dev))
        self.q_P = torch.nn.Parameter(torch.zeros((self.nblk_P, ntri), dtype=torch.float32, device=dev))
        # AdamW moments over the flat (q_R, q_P) batch and the updates since the last reset
        self.register_buffer("adam_m", torch.zeros((self.nblk, ntri), dtype=torch.float32, device=dev))
        self.register_buffer("adam_v", torch.zeros((self.nblk, ntri), dtype=torch.float32, device=dev))
        self.adam_t = 0

    @property
    def weight(self) -> torch.Tensor:
        """What the library reads as the stored weight: Wt, or the int8 buffer Wq."""
        return self.Wq if self.quantized else self.Wt

    def _desc(self, T: int) -> B.LinearDesc:
        variant = (B.POETX_MEM_Q8 if self.quantized else B.POETX_MEM if self.mem_efficient_mode
                   else B.POETX_FAST)
        return B.desc(T, self.out_features, self.in_features, self.block_size, self.k, _code(self.dtype), variant)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).to(self.dtype).contiguous()
        y = _PoetLinearFn.apply(x2, self.q_R, self.q_P, self)
        return y.reshape(*lead, self.out_features)

    @torch.no_grad()
    def optimizer_step(self, lr: float, gamma: float = 0.5, beta1: float = 0.9, beta2: float = 0.999,
                       eps: float = 1e-8, weight_decay: float = 0.0) -> None:
        """One AdamW update of q_R and q_P from their .grad at the rate lr * gamma
        (the POET learning-rate scaling); the gradients are left in place."""
        if self.q_R.grad is None or self.q_P.grad is None:
            raise RuntimeError("optimizer_step needs the gradients of q_R and q_P")
        q = torch.cat([self.q_R, self.q_P]).contiguous()
        g = torch.cat([self.q_R.grad, self.q_P.grad]).contiguous()
        self.adam_t += 1
        B.poetx_adamw_step(q, g, self.adam_m, self.adam_v, q.numel(), self.adam_t,
                           B.adamw_params(lr, gamma, beta1, beta2, eps, weight_decay))
        self.q_R.copy_(q[:self.nblk_R])
        self.q_P.copy_(q[self.nblk_R:])

    @torch.no_grad()
    def merge_then_reinitialize(self, generator: Optional[torch.Generator] = None) -> None:
        """Fold R W0 P into the stored weight, draw new permutations, set q to zero
        and reset the optimizer moments and count."""
        d = self._desc(0)
        pi_R_new = _perm(self.out_features, generator, self.weight.device)
        pi_P_new = _perm(self.in_features, generator, self.weight.device)
        ws = B.workspace(B.poetx_merge_workspace_bytes(d), self.weight.device)
        q_R = self.q_R.detach().contiguous()
        q_P = self.q_P.detach().contiguous()
        B.poetx_merge(d, self.weight, q_R, q_P, self.pi_R, self.pi_P, pi_R_new, pi_P_new, ws)
        self.q_R.copy_(q_R)
        self.q_P.copy_(q_P)
        self.pi_R.copy_(pi_R_new)
        self.pi_P.copy_(pi_P_new)
        B.poetx_adamw_reset(self.adam_m, self.adam_v, self.adam_m.numel())
        self.adam_t = 0
