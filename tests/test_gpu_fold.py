"""The R-side block product folded into the dense forward product
(poetx_dense_fold_r, and poetx_linear_fwd for bf16 chains with b = 256): z and
h2 must equal the dense product followed by the block product bit for bit, and
the layer's y must equal the unfused chain composed from the building blocks
(gather, block product, dense product, block product, scatter)."""
import numpy as np
import pytest
import torch

from orthogonal_equivalence_poet_amd import binding as B
from orthogonal_equivalence_poet_amd import inputs as I
from tests.gpu_helpers import DEV, dev, dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield
    torch.cuda.synchronize()


def _state(m, n, T, seed):
    spec = I.LinearSpec(f"fold_{m}x{n}_{T}", m=m, n=n, b=256, k=3, T=T, dtype="bf16", q_std=0.02, key=(71, seed, T))
    inp = I.make_linear_inputs(spec)
    nR, nP = m // 256, n // 256
    q = torch.cat([dev(inp["q_R"]), dev(inp["q_P"])]).contiguous()
    G = torch.empty((nR + nP, 256, 256), dtype=torch.bfloat16, device=DEV)
    B.poetx_cnp_fwd(q, nR + nP, 256, 3, G, B.workspace(B.poetx_cnp_fwd_workspace_bytes(nR + nP, 256, 3,
                                                                                       B.POETX_BF16)))
    Wt = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    B.poetx_prepermute(dev(inp["W0"], "bf16"), Wt, m, n, dev_i32(inp["pi_R"]), dev_i32(inp["pi_P"]))
    return spec, inp, G[:nR], G[nR:], Wt


SHAPES = [(4096, 4096, 2048),   # the q_proj shape: one 128 x 256 tile per CU
          (512, 256, 300),      # ragged last token tile
          (768, 1024, 77),
          (256, 512, 1)]


@pytest.mark.parametrize("m,n,T", SHAPES)
def test_dense_fold_r_equals_dense_then_block_product(m, n, T):
    _, inp, G_R, _, Wt = _state(m, n, T, 1)
    h1 = dev(inp["x"], "bf16")          # any bf16 input of the shape
    h2_ref = torch.empty((T, m), dtype=torch.bfloat16, device=DEV)
    z_ref = torch.empty_like(h2_ref)
    B.poetx_gemm(B.POETX_GEMM_NT, h1, Wt, h2_ref, T, m, n, dense=True)
    B.poetx_block_apply(h2_ref, G_R, z_ref, T, m, 256)
    h2 = torch.full_like(h2_ref, float("nan"))
    z = torch.full_like(h2_ref, float("nan"))
    B.poetx_dense_fold_r(h1, Wt, G_R, z, T, m, n, 256, h2=h2)
    assert torch.equal(h2, h2_ref)
    assert torch.equal(z, z_ref)
    z2 = torch.full_like(h2_ref, float("nan"))
    B.poetx_dense_fold_r(h1, Wt, G_R, z2, T, m, n, 256)     # without h2
    assert torch.equal(z2, z_ref)


# layer shapes whose 128 x 256 tile grid the forward folds (a multiple of 256
# tiles), with ragged last token tiles, and one it does not
LAYER_SHAPES = [(4096, 4096, 2048), (4096, 1024, 2000), (1024, 512, 8100), (768, 1024, 77)]


@pytest.mark.parametrize("variant", [B.POETX_FAST, B.POETX_MEM])
@pytest.mark.parametrize("m,n,T", LAYER_SHAPES)
def test_layer_forward_equals_unfused_chain(variant, m, n, T):
    spec, inp, G_R, G_P, Wt = _state(m, n, T, 2)
    x = dev(inp["x"], "bf16")
    pi_R, pi_P = dev_i32(inp["pi_R"]), dev_i32(inp["pi_P"])
    # the unfused chain from the building blocks
    a = torch.empty((T, n), dtype=torch.bfloat16, device=DEV)
    h1 = torch.empty_like(a)
    h2 = torch.empty((T, m), dtype=torch.bfloat16, device=DEV)
    zz = torch.empty_like(h2)
    y_ref = torch.empty_like(h2)
    B.poetx_permute(x, a, T, n, col_idx=pi_P)
    B.poetx_block_apply(a, G_P, h1, T, n, 256)
    B.poetx_gemm(B.POETX_GEMM_NT, h1, Wt, h2, T, m, n, dense=True)
    B.poetx_block_apply(h2, G_R, zz, T, m, 256)
    B.poetx_permute(zz, y_ref, T, m, col_idx=pi_R, scatter_cols=True)
    d = B.desc(T, m, n, 256, 3, B.POETX_BF16, variant)
    y = torch.full_like(y_ref, float("nan"))
    saved = B.workspace(B.poetx_linear_saved_bytes(d))
    ws = B.workspace(B.poetx_linear_fwd_workspace_bytes(d))
    for _ in range(2):
        B.poetx_linear_fwd(d, x, Wt, G_R, G_P, pi_R, pi_P, y, saved, ws)
        assert torch.equal(y, y_ref)
    if variant == B.POETX_FAST:    # the kept h2 and gathered input feed the backward
        kept = saved[: T * m * 2].view(torch.bfloat16).view(T, m)
        assert torch.equal(kept, h2)
    assert np.isfinite(y.float().cpu().numpy()).all()
