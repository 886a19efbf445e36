"""poetx_linear_fwd_noalloc (the forward for callers that cannot allocate)
against poetx_linear_fwd with a caller workspace: two calls in a row on the
library's scratch array, the second smaller, each bit-identical to the
workspace entry point (the same kernels on the same values); and a descriptor
beyond the array's size is refused before any launch."""
import numpy as np
import pytest
import torch

from orthogonal_equivalence_poet_amd import binding as B
from orthogonal_equivalence_poet_amd import inputs as I
from tests.gpu_helpers import GpuLayer, cnp_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield
    torch.cuda.synchronize()


def _both(spec, variant):
    inp = I.make_linear_inputs(spec)
    g = GpuLayer(spec, inp, variant)
    s = spec
    G_R = cnp_fwd(g.q_R, s.nblk_R, s.b, s.k, s.dtype)
    G_P = cnp_fwd(g.q_P, s.nblk_P, s.b, s.k, s.dtype)
    nsaved = B.poetx_linear_saved_bytes(g.desc)
    assert B.poetx_linear_fwd_workspace_bytes(g.desc) <= B.POETX_NOALLOC_SCRATCH_BYTES
    y_ref = torch.empty((s.T, s.m), dtype=g.x.dtype, device="cuda")
    y = torch.full_like(y_ref, 7.0)
    saved_ref = B.workspace(nsaved)
    saved = B.workspace(nsaved)
    if saved is not None:
        saved.fill_(0x5A)
    ws = B.workspace(B.poetx_linear_fwd_workspace_bytes(g.desc))
    B.poetx_linear_fwd(g.desc, g.x, g.weight, G_R, G_P, g.pi_R, g.pi_P, y_ref, saved_ref, ws)
    B.poetx_linear_fwd_noalloc(g.desc, g.x, g.weight, G_R, G_P, g.pi_R, g.pi_P, y, saved)
    torch.cuda.synchronize()
    return y, y_ref, saved, saved_ref


def test_noalloc_forward_twice_second_smaller_matches_workspace_forward():
    # first: the Llama-8B q_proj-shaped fast forward (33.6 MB of scratch)
    big = I.LinearSpec("noalloc_big", m=4096, n=4096, b=256, k=3, T=2048, dtype="bf16", q_std=1e-3,
                       key=(31, 0, 0))
    y, y_ref, saved, saved_ref = _both(big, "fast")
    assert torch.equal(y, y_ref)
    assert torch.equal(saved, saved_ref)
    # second, smaller and ragged, mem variant, on the same scratch right after
    small = I.LinearSpec("noalloc_small", m=768, n=512, b=128, k=3, T=300, dtype="bf16", q_std=0.02,
                         key=(31, 1, 0))
    y, y_ref, _, _ = _both(small, "mem")
    assert torch.equal(y, y_ref)
    # and a float32 fast one
    tiny = I.tiny()
    y, y_ref, saved, saved_ref = _both(tiny, "fast")
    assert torch.equal(y, y_ref) and torch.equal(saved, saved_ref)


def test_noalloc_forward_refuses_sizes_beyond_its_scratch():
    d = B.desc(8192, 14336, 4096, 512, 4, B.POETX_BF16, B.POETX_MEM)
    assert B.poetx_linear_fwd_workspace_bytes(d) > B.POETX_NOALLOC_SCRATCH_BYTES
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")   # never read: refused first
    with pytest.raises(B.PoetxError) as e:
        B.poetx_linear_fwd_noalloc(d, x, x, x, x, x, x, x, None)
    assert e.value.status == B.POETX_ERR_WORKSPACE
