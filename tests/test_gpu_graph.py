"""The whole training step (Cayley-Neumann forward keeping its intermediates,
layer forward and backward, Cayley-Neumann backward, AdamW update) captured in
a HIP graph: the library allocates nothing and records no memset nodes, so a
graph of its calls replays to the same bytes as the eager calls.  Each replay
is checked against eager work done between the replays."""
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


@pytest.mark.parametrize("dtype,variant", [("f32", B.POETX_FAST), ("bf16", B.POETX_MEM), ("bf16", B.POETX_FAST),
                                           ("bf16", B.POETX_MEM_Q8), ("bf16", B.POETX_FOUR_PERM),
                                           ("bf16", B.POETX_WEIGHT_CENTRIC)])
def test_step_graph_replays_match_eager(dtype, variant):
    T, m, n, b, k = 96, 256, 128, 64, 3
    spec = I.LinearSpec("graph", m=m, n=n, b=b, k=k, T=T, dtype=dtype, q_std=0.02, key=(13, m, n))
    inp = I.make_linear_inputs(spec)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    code = B.POETX_F32 if dtype == "f32" else B.POETX_BF16
    d = B.desc(T, m, n, b, k, code, variant)
    nblk = m // b + n // b
    x, dy = dev(inp["x"], dtype), dev(inp["dy"], dtype)
    pi_R, pi_P = dev_i32(inp["pi_R"]), dev_i32(inp["pi_P"])
    Wt = torch.empty((m, n), dtype=td, device=DEV)
    B.poetx_prepermute(dev(inp["W0"], dtype), Wt, m, n, pi_R, pi_P)
    if variant == B.POETX_MEM_Q8:        # the int8 storage of the pre-permuted weight
        Wq = B.workspace(B.poetx_qweight_bytes(m, n))
        B.poetx_quantize_weight(Wt, m, n, Wq)
        Wt = Wq
    elif variant in (B.POETX_FOUR_PERM, B.POETX_WEIGHT_CENTRIC):   # these take W0 itself
        Wt = dev(inp["W0"], dtype)
    q0 = torch.cat([dev(inp["q_R"]), dev(inp["q_P"])]).contiguous()
    q = q0.clone()
    G = torch.empty((nblk, b, b), dtype=td, device=DEV)
    dG = torch.empty((nblk, b, b), dtype=torch.float32, device=DEV)
    dq = torch.empty_like(q)
    mom, vel = torch.zeros_like(q), torch.zeros_like(q)
    y = torch.empty((T, m), dtype=td, device=DEV)
    dx = torch.empty((T, n), dtype=td, device=DEV)
    saved = B.workspace(B.poetx_linear_saved_bytes(d))
    ws = B.workspace(max(B.poetx_linear_fwd_workspace_bytes(d), B.poetx_linear_bwd_workspace_bytes(d),
                         B.poetx_cnp_fwd_workspace_bytes(nblk, b, k, code),
                         B.poetx_cnp_bwd_workspace_bytes(nblk, b, k, code)))
    cnp_saved = B.workspace(B.poetx_cnp_saved_bytes(nblk, b, k, code))
    opt = B.adamw_params(1e-3)
    count = q.numel()

    def step():
        B.poetx_cnp_fwd_save(q, nblk, b, k, G, cnp_saved, ws)
        B.poetx_linear_fwd(d, x, Wt, G[:m // b], G[m // b:], pi_R, pi_P, y, saved, ws)
        B.poetx_linear_bwd(d, dy, x, Wt, G[:m // b], G[m // b:], pi_R, pi_P, saved, dx, dG[:m // b], dG[m // b:], ws)
        B.poetx_cnp_bwd_saved(q, dG, nblk, b, k, dq, code, cnp_saved, ws)
        B.poetx_adamw_step(q, dq, mom, vel, count, 1, opt)

    def reset():
        q.copy_(q0)
        mom.zero_()
        vel.zero_()

    outs = (y, dx, dG, dq, q, mom, vel)
    reset()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        for t in (y, dx, dG, dq):
            t.fill_(float("nan"))
        reset()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want)
        reset()
        step()   # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(q, ref[4])
    assert np.isfinite(ref[3].cpu().numpy()).all()


def test_group_step_graph_replays_match_eager():
    """q/k/v-shaped group (grouped dense launches), mem variant, captured and replayed."""
    T, n, b, k = 130, 256, 64, 3
    ms = [256, 128, 128]
    specs = [I.LinearSpec(f"ggraph{i}", m=m, n=n, b=b, k=k, T=T, dtype="bf16", q_std=0.02, key=(14, i, m))
             for i, m in enumerate(ms)]
    inps = [I.make_linear_inputs(sp) for sp in specs]
    M = sum(ms)
    x = dev(inps[0]["x"], "bf16")
    dy = torch.cat([dev(inp["dy"], "bf16") for inp in inps], dim=1).contiguous()
    pi_R = torch.cat([dev_i32(inp["pi_R"]) for inp in inps]).contiguous()
    pi_P = torch.cat([dev_i32(inp["pi_P"]) for inp in inps]).contiguous()
    Wt = torch.empty((M, n), dtype=torch.bfloat16, device=DEV)
    o = 0
    for m, inp, pr, pp in zip(ms, inps, pi_R.split(ms), pi_P.split(n)):
        B.poetx_prepermute(dev(inp["W0"], "bf16"), Wt[o:o + m], m, n, pr, pp)
        o += m
    qR = torch.cat([dev(inp["q_R"]) for inp in inps])
    qP = torch.cat([dev(inp["q_P"]) for inp in inps])
    q = torch.cat([qR, qP]).contiguous()
    nR, nblk = M // b, M // b + len(ms) * n // b
    G = torch.empty((nblk, b, b), dtype=torch.bfloat16, device=DEV)
    dG = torch.empty((nblk, b, b), dtype=torch.float32, device=DEV)
    dq = torch.empty_like(q)
    y = torch.empty((T, M), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty((T, n), dtype=torch.bfloat16, device=DEV)
    gd = B.group_desc(T, n, b, k, B.POETX_BF16, B.POETX_MEM, ms)
    ws = B.workspace(max(B.poetx_group_fwd_workspace_bytes(gd), B.poetx_group_bwd_workspace_bytes(gd),
                         B.poetx_cnp_fwd_workspace_bytes(nblk, b, k, B.POETX_BF16),
                         B.poetx_cnp_bwd_workspace_bytes(nblk, b, k, B.POETX_BF16)))
    cnp_saved = B.workspace(B.poetx_cnp_saved_bytes(nblk, b, k, B.POETX_BF16))

    def step():
        B.poetx_cnp_fwd_save(q, nblk, b, k, G, cnp_saved, ws)
        B.poetx_group_fwd(gd, x, Wt, G[:nR], G[nR:], pi_R, pi_P, y, None, ws)
        B.poetx_group_bwd(gd, dy, x, Wt, G[:nR], G[nR:], pi_R, pi_P, None, dx, dG[:nR], dG[nR:], ws)
        B.poetx_cnp_bwd_saved(q, dG, nblk, b, k, dq, B.POETX_BF16, cnp_saved, ws)

    outs = (y, dx, dG, dq)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        for t in outs:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want)
        step()   # eager work between the replays
        torch.cuda.synchronize()
    assert np.isfinite(ref[3].cpu().numpy()).all()
