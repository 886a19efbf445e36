"""GPU parity: libpoetx through its C ABI against the float64 oracle on the
same seeded inputs.  Data movement (skew layout, permutations, merge index
maps) must be bit-exact; floating point is held to a relative Frobenius error
of 1e-5 (float32 path) or 1.5e-2 (bf16 operands, float32 accumulation)."""
import numpy as np
import pytest
import torch

from oracle import poet_oracle as O
from orthogonal_equivalence_poet_amd import binding as B
from orthogonal_equivalence_poet_amd import inputs as I
from tests.gpu_helpers import (DEV, GpuLayer, cnp_bwd, cnp_fwd, code, dev, dev_i32, host, rel_fro, tdtype,
                               tol)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield
    torch.cuda.synchronize()


def _q(nblk, b, std, seed):
    return I.gaussian((nblk, b * (b - 1) // 2), std, "f32", 90, seed)


# ------------------------------------------------------------ skew storage
@pytest.mark.parametrize("b", [16, 48, 64, 256, 512])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_skew_unpack_bitexact(b, dtype):
    nblk = 3
    q = _q(nblk, b, 1.0, b)
    Q = torch.empty((nblk, b, b), dtype=tdtype(dtype), device=DEV)
    B.poetx_skew_unpack(dev(q), Q, nblk, b)
    ref = O.skew_from_params(q, b).astype(np.float32)
    if dtype == "bf16":
        ref = I.round_to_bf16(ref)
    assert np.array_equal(host(Q), ref.astype(np.float64))


@pytest.mark.parametrize("b", [16, 48, 256])
def test_skew_pack_bitexact(b):
    nblk = 4
    dQ = I.gaussian((nblk, b, b), 1.0, "f32", 91, b)
    dq = torch.empty((nblk, b * (b - 1) // 2), dtype=torch.float32, device=DEV)
    B.poetx_skew_pack(dev(dQ), dq, nblk, b)
    ref = O.params_grad_from_skew_grad(dQ).astype(np.float32)   # one correctly rounded subtraction
    assert np.array_equal(host(dq), ref.astype(np.float64))


# ------------------------------------------------------------ permutations
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
# rows of 16 B to 57 KB in LDS (each thread's share of a row's 16-byte vectors
# 1 to 14: batches of 2, 4 and 8, one or several per row) and rows past LDS
@pytest.mark.parametrize("rows,cols", [(37, 4096), (3, 16), (300, 512), (9, 6144), (5, 14336), (2, 40960)])
@pytest.mark.parametrize("mode", ["gather", "scatter", "rows_and_cols"])
def test_permute_bitexact(dtype, rows, cols, mode):
    src = I.gaussian((rows, cols), 1.0, dtype, 92, rows, cols)
    pc = I.permutation(cols, 93, cols)
    pr = I.permutation(rows, 94, rows)
    dst = torch.empty((rows, cols), dtype=tdtype(dtype), device=DEV)
    if mode == "gather":
        B.poetx_permute(dev(src, dtype), dst, rows, cols, None, dev_i32(pc), False)
        ref = src[:, pc]
    elif mode == "scatter":
        B.poetx_permute(dev(src, dtype), dst, rows, cols, None, dev_i32(pc), True)
        ref = np.empty_like(src)
        ref[:, pc] = src
    else:
        B.poetx_permute(dev(src, dtype), dst, rows, cols, dev_i32(pr), dev_i32(pc), False)
        ref = src[pr][:, pc]
    assert np.array_equal(host(dst), ref.astype(np.float64))


def test_prepermute_bitexact():
    spec = I.llama8b_q_proj()
    m, n = 512, 1024
    W0 = I.gaussian((m, n), 0.02, "bf16", 95)
    pr, pc = I.permutation(m, 96), I.permutation(n, 97)
    Wt = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    B.poetx_prepermute(dev(W0, "bf16"), Wt, m, n, dev_i32(pr), dev_i32(pc))
    assert np.array_equal(host(Wt), O.prepermute(W0, pr, pc))
    del spec


def test_check_perm():
    n = 1000
    pi = I.permutation(n, 98)
    ok = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = B.workspace(B.poetx_check_perm_workspace_bytes(n))
    B.poetx_check_perm(dev_i32(pi), n, ok, ws)
    assert int(ok.item()) == 1
    bad = pi.copy()
    bad[5] = bad[6]
    B.poetx_check_perm(dev_i32(bad), n, ok, ws)
    assert int(ok.item()) == 0
    bad = pi.copy()
    bad[0] = n + 3
    B.poetx_check_perm(dev_i32(bad), n, ok, ws)
    assert int(ok.item()) == 0


# -------------------------------------------------- Cayley-Neumann transform
CNP_CASES = [
    # b, k, dtype, std, target block norm
    (16, 3, "f32", 0.05, None),
    (16, 3, "bf16", 0.05, None),
    (48, 3, "f32", 0.05, None),
    (64, 1, "f32", 0.05, None),
    (64, 2, "f32", 0.05, None),
    (64, 5, "f32", 0.05, None),
    (64, 6, "bf16", 0.05, None),
    (128, 4, "f32", 1e-2, 0.5),
    (256, 3, "f32", 1e-3, None),
    (256, 3, "bf16", 1e-3, None),
    (256, 3, "bf16", 1e-2, 0.7),
    (128, 3, "bf16", 0.05, None),
    (128, 2, "bf16", 1e-2, 0.5),
    (64, 3, "bf16", 0.05, None),
    (512, 3, "bf16", 1e-2, 0.5),
    (512, 4, "bf16", 1e-2, 0.5),
    (512, 4, "f32", 1e-2, 0.5),
]


def _scaled_q(nblk, b, std, norm, seed):
    q = _q(nblk, b, std, seed)
    if norm is not None:
        Q = O.skew_from_params(q, b)
        for j in range(nblk):
            q[j] *= norm / np.linalg.norm(Q[j], 2)
    return q.astype(np.float32)


@pytest.mark.parametrize("b,k,dtype,std,norm", CNP_CASES)
def test_cnp_fwd_parity(b, k, dtype, std, norm):
    nblk = 5
    q = _scaled_q(nblk, b, std, norm, 200 + b + k)
    G = host(cnp_fwd(dev(q), nblk, b, k, dtype))
    ref = O.neumann_cayley(O.skew_from_params(q, b), k)
    assert rel_fro(G, ref) <= tol(dtype)
    eye = np.eye(b)
    # the informative part G - I (small for small q) is checked on its own.
    # Against the exact G, bf16 storage alone costs up to 1.62e-2 here (at
    # b = 256, q ~ N(0, 1e-3^2) the diagonal 1 - 2.6e-4 rounds to 1.0, and G - I
    # loses its diagonal), so that check is held to 3e-2; against the oracle's G
    # rounded to bf16 once (the best a bf16 output can be) it meets the bf16 bar.
    assert rel_fro(G - eye, ref - eye) <= (1e-4 if dtype == "f32" else 3e-2)
    if dtype == "bf16":
        ref_bf = I.round_to_bf16(ref.astype(np.float32)).astype(np.float64)
        assert rel_fro(G - eye, ref_bf - eye) <= tol(dtype)


@pytest.mark.parametrize("b,k,dtype,std,norm", CNP_CASES)
def test_cnp_bwd_parity(b, k, dtype, std, norm):
    nblk = 5
    q = _scaled_q(nblk, b, std, norm, 300 + b + k)
    dG = I.gaussian((nblk, b, b), 1.0, "f32", 301, b, k)
    dq = host(cnp_bwd(dev(q), dev(dG), nblk, b, k, dtype))
    ref = O.params_grad_from_skew_grad(O.cnp_vjp(O.skew_from_params(q, b), dG, k))
    assert rel_fro(dq, ref) <= tol(dtype)


# b = 256, k = 3, bf16 batches of 144 blocks or more take the one-block-per-
# workgroup backward (below that, the passes over tile units); a sample of
# blocks, among them the first and last of a ragged count, against the oracle
@pytest.mark.parametrize("nblk,std,norm", [(143, 1e-2, 0.5), (150, 1e-2, 0.5), (256, 1e-3, None),
                                           (300, 1e-2, None), (517, 1e-2, 0.6)])
def test_cnp_bwd_many_blocks(nblk, std, norm):
    b, k = 256, 3
    q = _q(nblk, b, std, 600 + nblk)
    js = [0, 1, nblk // 2, nblk - 1]
    if norm is not None:
        q[js] = _scaled_q(len(js), b, std, norm, 601 + nblk)
    dG = I.gaussian((nblk, b, b), 1.0, "f32", 602, nblk)
    dq = host(cnp_bwd(dev(q), dev(dG), nblk, b, k, "bf16")[js])
    ref = O.params_grad_from_skew_grad(O.cnp_vjp(O.skew_from_params(q[js], b), dG[js], k))
    assert rel_fro(dq, ref) <= tol("bf16")    # every sampled block on its own, too


# dG and G off 16-byte alignment (a view at an odd element offset): the fused
# and per-block kernels need 16-byte rows, so these calls take the general
# b x b products; their results must be the same transform
@pytest.mark.parametrize("nblk", [32, 150])
def test_cnp_unaligned_buffers_take_general_path(nblk):
    b, k = 256, 3
    q = _q(nblk, b, 1e-2, 700 + nblk)
    js = [0, nblk // 2, nblk - 1]
    dG = I.gaussian((nblk, b, b), 1.0, "f32", 701, nblk)
    dG_buf = torch.empty(nblk * b * b + 1, dtype=torch.float32, device=DEV)
    dG_view = dG_buf[1:].view(nblk, b, b)              # 4 bytes past a 16-byte boundary
    dG_view.copy_(dev(dG))
    dq = host(cnp_bwd(dev(q), dG_view, nblk, b, k, "bf16")[js])
    ref = O.params_grad_from_skew_grad(O.cnp_vjp(O.skew_from_params(q[js], b), dG[js], k))
    assert rel_fro(dq, ref) <= tol("bf16")
    G_buf = torch.empty(nblk * b * b + 1, dtype=torch.bfloat16, device=DEV)
    G = G_buf[1:].view(nblk, b, b)                      # 2 bytes past a 16-byte boundary
    ws = B.workspace(B.poetx_cnp_fwd_workspace_bytes(nblk, b, k, B.POETX_BF16))
    B.poetx_cnp_fwd(dev(q), nblk, b, k, G, ws)
    ref_G = O.neumann_cayley(O.skew_from_params(q[js], b), k)
    assert rel_fro(host(G[js]), ref_G) <= tol("bf16")


# bf16 blocks of 128 or 256 take the fused per-panel forward (32-row panels for
# a few blocks, as in the cases above; 64-row panels once there are 256 or more
# of those), except k = 3 at b = 256 from 96 blocks on, which takes one block
# per workgroup; here many blocks, a sample of which is checked against the oracle.
@pytest.mark.parametrize("b,k,std,norm,nblk", [(256, 3, 1e-3, None, 256), (256, 1, 0.05, None, 256),
                                               (256, 4, 1e-2, 0.5, 256), (256, 7, 1e-2, 0.6, 256),
                                               (128, 3, 0.05, None, 512), (128, 2, 1e-2, 0.5, 512),
                                               (256, 3, 1e-3, None, 1024), (256, 4, 1e-2, 0.5, 1100),
                                               (256, 3, 1e-2, 0.6, 97), (256, 3, 1e-2, None, 95)])
def test_cnp_fused_forward_many_blocks(b, k, std, norm, nblk):
    # many blocks, including ragged block counts on both sides of the k = 3 switch
    q = _q(nblk, b, std, 500 + b + k)
    js = [0, 1, nblk // 2, nblk - 1]
    if norm is not None:
        q[js] = _scaled_q(len(js), b, std, norm, 501 + b + k)
    G = host(cnp_fwd(dev(q), nblk, b, k, "bf16")[js])
    ref = O.blocks_from_params(q[js], b, k)
    assert rel_fro(G, ref) <= tol("bf16")


@pytest.mark.parametrize("b,k,dtype,nblk", [(256, 3, "bf16", 6), (256, 3, "bf16", 256), (256, 3, "bf16", 1030),
                                            (128, 3, "bf16", 512),
                                            (64, 3, "f32", 6), (128, 4, "bf16", 6), (128, 4, "bf16", 512),
                                            (64, 5, "bf16", 6), (16, 2, "f32", 6), (64, 4, "f32", 6),
                                            (512, 4, "bf16", 36)])
def test_cnp_saved_variant_is_bitwise_identical(b, k, dtype, nblk):
    """Forward keeping the square and its companions, backward reusing them:
    the same products on the same values as the recomputing pair."""
    q = dev(_q(nblk, b, 0.05, 400 + b + k))
    dG = dev(I.gaussian((nblk, b, b), 1.0, "f32", 401, b, k))
    G_ref = cnp_fwd(q, nblk, b, k, dtype)
    dq_ref = cnp_bwd(q, dG, nblk, b, k, dtype)
    saved = B.workspace(B.poetx_cnp_saved_bytes(nblk, b, k, code(dtype)))
    G = torch.empty_like(G_ref)
    ws = B.workspace(B.poetx_cnp_bwd_workspace_bytes(nblk, b, k, code(dtype)))
    B.poetx_cnp_fwd_save(q, nblk, b, k, G, saved, ws)
    dq = torch.empty_like(dq_ref)
    B.poetx_cnp_bwd_saved(q, dG, nblk, b, k, dq, code(dtype), saved, ws)
    # bf16 blocks of 128 / 256 take a fused forward (per panel, or per block for
    # k = 3 at b = 256 from 96 blocks on); the saving forward does so only for
    # k = 3 (for other k the backward needs the square's float32 companions)
    fused_plain = dtype == "bf16" and b in (128, 256)
    fused_save = fused_plain and k == 3
    js = [0, nblk - 1]
    if fused_plain == fused_save:
        assert torch.equal(G, G_ref)
    else:
        G_or = O.blocks_from_params(host(q[js]), b, k)
        assert rel_fro(host(G[js]), G_or) <= tol(dtype) and rel_fro(host(G_ref[js]), G_or) <= tol(dtype)
    if fused_save:
        # the fused forward keeps Q, S and 2Q + S as it formed them on chip, the
        # recomputing backward re-derives them through the square product:
        # both are the same values up to bf16 rounding
        ref = O.params_grad_from_skew_grad(O.cnp_vjp(O.skew_from_params(host(q[js]), b), host(dG[js]), k))
        assert rel_fro(host(dq[js]), ref) <= tol(dtype)
        assert rel_fro(host(dq), host(dq_ref)) <= tol(dtype)
    else:
        assert torch.equal(dq, dq_ref)


# ------------------------------------------------------------------ layer
def _oracle_step(spec, inp):
    G_R = O.blocks_from_params(inp["q_R"], spec.b, spec.k)
    G_P = O.blocks_from_params(inp["q_P"], spec.b, spec.k)
    y = O.forward_from_blocks(inp["x"], inp["W0"], G_R, G_P, inp["pi_R"], inp["pi_P"])
    dx, dq_R, dq_P, dG_R, dG_P = O.backward(inp["dy"], inp["x"], inp["W0"], inp["q_R"], inp["q_P"],
                                            inp["pi_R"], inp["pi_P"], spec.b, spec.k)
    return dict(y=y, dx=dx, dq_R=dq_R, dq_P=dq_P, dG_R=dG_R, dG_P=dG_P, G_R=G_R, G_P=G_P)


def _check_step(g, ref, dtype):
    t = tol(dtype)
    got = dict(y=host(g.y), dx=host(g.dx), dq_R=host(g.dq_R), dq_P=host(g.dq_P), dG_R=host(g.dG_R),
               dG_P=host(g.dG_P), G_R=host(g.G_R), G_P=host(g.G_P))
    errs = {k: rel_fro(got[k], ref[k]) for k in got}
    bad = {k: v for k, v in errs.items() if v > t}
    assert not bad, errs


@pytest.mark.parametrize("variant", ["fast", "mem"])
def test_tiny_fp32_layer(variant):
    spec = I.tiny()
    inp = I.make_linear_inputs(spec)
    g = GpuLayer(spec, inp, variant)
    g.forward()
    g.backward()
    _check_step(g, _oracle_step(spec, inp), "f32")


RAGGED = [
    # m, n, b, k, T, dtype
    (768, 512, 128, 3, 300, "bf16"),
    (768, 512, 128, 3, 300, "f32"),
    (512, 1024, 256, 3, 257, "bf16"),
    (256, 768, 256, 4, 129, "bf16"),
    (96, 160, 32, 2, 77, "f32"),
    (64, 64, 16, 5, 1, "f32"),
]


@pytest.mark.parametrize("m,n,b,k,T,dtype", RAGGED)
@pytest.mark.parametrize("variant", ["fast", "mem"])
def test_layer_ragged(m, n, b, k, T, dtype, variant):
    spec = I.LinearSpec(f"ragged_{m}x{n}", m=m, n=n, b=b, k=k, T=T, dtype=dtype, q_std=0.02, key=(7, m, T))
    inp = I.make_linear_inputs(spec)
    g = GpuLayer(spec, inp, variant)
    g.forward()
    g.backward()
    _check_step(g, _oracle_step(spec, inp), dtype)


# The comparison variants (all four permutations on the activations; the
# original weight-centric POET with dense R and P) against the same oracle.
@pytest.mark.parametrize("m,n,b,k,T,dtype", RAGGED + [(64, 48, 16, 3, 40, "bf16"), (1024, 512, 256, 3, 2048, "bf16")])
@pytest.mark.parametrize("variant", ["four_perm", "weight_centric"])
def test_comparison_variants_ragged(m, n, b, k, T, dtype, variant):
    spec = I.LinearSpec(f"cmp_{m}x{n}", m=m, n=n, b=b, k=k, T=T, dtype=dtype, q_std=0.02, key=(17, m, T))
    inp = I.make_linear_inputs(spec)
    g = GpuLayer(spec, inp, variant)
    g.forward()
    g.backward()
    _check_step(g, _oracle_step(spec, inp), dtype)


@pytest.mark.parametrize("variant", ["four_perm", "weight_centric"])
def test_comparison_variants_tiny_and_deterministic(variant):
    spec = I.tiny()
    inp = I.make_linear_inputs(spec)
    outs = []
    for _ in range(2):
        g = GpuLayer(spec, inp, variant)
        g.forward()
        g.backward()
        outs.append([t.clone() for t in (g.y, g.dx, g.dG_R, g.dG_P)])
    _check_step(g, _oracle_step(spec, inp), "f32")
    for a, c in zip(*outs):
        assert torch.equal(a, c)


def test_comparison_variants_empty_batch():
    spec = I.LinearSpec("empty_cmp", m=256, n=128, b=64, k=3, T=0, dtype="bf16", key=(18, 0, 0))
    inp = I.make_linear_inputs(spec)
    for variant in ("four_perm", "weight_centric"):
        g = GpuLayer(spec, inp, variant)
        g.forward()
        g.dG_R = torch.full((4, 64, 64), 7.0, device=DEV)
        g.dG_P = torch.full((2, 64, 64), 7.0, device=DEV)
        ws = B.workspace(B.poetx_linear_bwd_workspace_bytes(g.desc))
        B.poetx_linear_bwd(g.desc, g.dy, g.x, g.weight, g.G_R, g.G_P, g.pi_R, g.pi_P, g.saved, g.x, g.dG_R,
                           g.dG_P, ws)
        assert not g.dG_R.any() and not g.dG_P.any()


def test_fast_and_mem_agree_bitwise_and_runs_are_deterministic():
    spec = I.LinearSpec("det", m=1024, n=512, b=256, k=3, T=700, dtype="bf16", key=(8, 0, 0))
    inp = I.make_linear_inputs(spec)
    outs = []
    for variant in ("fast", "mem", "fast"):
        g = GpuLayer(spec, inp, variant)
        g.forward()
        g.backward()
        outs.append([t.clone() for t in (g.y, g.dx, g.dG_R, g.dG_P, g.dq_R, g.dq_P)])
    for a, b_, c in zip(*outs):
        assert torch.equal(a, b_) and torch.equal(a, c)


def test_empty_batch_gives_zero_block_gradients():
    spec = I.LinearSpec("empty", m=256, n=256, b=64, k=3, T=0, dtype="bf16", key=(9, 0, 0))
    inp = I.make_linear_inputs(spec)
    g = GpuLayer(spec, inp, "fast")
    g.forward()
    g.dG_R = torch.full((4, 64, 64), 7.0, device=DEV)
    g.dG_P = torch.full((4, 64, 64), 7.0, device=DEV)
    ws = B.workspace(B.poetx_linear_bwd_workspace_bytes(g.desc))
    B.poetx_linear_bwd(g.desc, g.dy, g.x, g.Wt, g.G_R, g.G_P, g.pi_R, g.pi_P, g.saved, g.x, g.dG_R, g.dG_P, ws)
    assert not g.dG_R.any() and not g.dG_P.any()


def test_q_zero_layer_is_plain_linear():
    spec = I.LinearSpec("qzero", m=512, n=256, b=128, k=3, T=64, dtype="f32", key=(10, 0, 0))
    inp = I.make_linear_inputs(spec)
    inp["q_R"][:] = 0
    inp["q_P"][:] = 0
    g = GpuLayer(spec, inp, "fast")
    y = host(g.forward())
    assert rel_fro(y, inp["x"].astype(np.float64) @ inp["W0"].astype(np.float64).T) <= 1e-6


# ------------------------------------------------------------------ merge
def _merge(g, pi_R_new, pi_P_new):
    ws = B.workspace(B.poetx_merge_workspace_bytes(g.desc))
    B.poetx_merge(g.desc, g.Wt, g.q_R, g.q_P, g.pi_R, g.pi_P, pi_R_new, pi_P_new, ws)


@pytest.mark.parametrize("m,n,b,k,dtype", [(64, 64, 16, 3, "f32"), (512, 256, 128, 3, "bf16"),
                                           (512, 1024, 256, 4, "bf16")])
def test_merge_parity(m, n, b, k, dtype):
    spec = I.LinearSpec("merge", m=m, n=n, b=b, k=k, T=16, dtype=dtype, q_std=0.05, key=(11, m, n))
    inp = I.make_linear_inputs(spec, with_new_perm=True)
    g = GpuLayer(spec, inp, "fast")
    Wt0 = O.prepermute(inp["W0"], inp["pi_R"], inp["pi_P"])
    _merge(g, dev_i32(inp["pi_R_new"]), dev_i32(inp["pi_P_new"]))
    ref, _, _ = O.merge(Wt0, inp["q_R"], inp["q_P"], inp["pi_R"], inp["pi_P"], inp["pi_R_new"], inp["pi_P_new"],
                        b, k)
    assert rel_fro(host(g.Wt), ref) <= tol(dtype)
    assert not g.q_R.any() and not g.q_P.any()


def test_merge_with_zero_q_and_same_perms_is_bitexact_noop():
    spec = I.LinearSpec("noop", m=512, n=1024, b=256, k=3, T=16, dtype="bf16", key=(12, 0, 0))
    inp = I.make_linear_inputs(spec)
    inp["q_R"][:] = 0
    inp["q_P"][:] = 0
    g = GpuLayer(spec, inp, "fast")
    before = g.Wt.clone()
    _merge(g, g.pi_R, g.pi_P)
    assert torch.equal(before, g.Wt)


def test_merge_preserves_layer_output():
    spec = I.LinearSpec("inv", m=1024, n=512, b=128, k=3, T=200, dtype="f32", q_std=0.05, key=(13, 0, 0))
    inp = I.make_linear_inputs(spec, with_new_perm=True)
    g = GpuLayer(spec, inp, "fast")
    y0 = host(g.forward())
    _merge(g, dev_i32(inp["pi_R_new"]), dev_i32(inp["pi_P_new"]))
    g.pi_R = dev_i32(inp["pi_R_new"])
    g.pi_P = dev_i32(inp["pi_P_new"])
    y1 = host(g.forward())
    assert rel_fro(y1, y0) <= 1e-5


# --------------------------------------------------------- building blocks
GEMM_CASES = [
    # layout, dense, M, N, K, dtype
    ("NT", True, 2048, 4096, 4096, "bf16"),
    ("NN", True, 2048, 4096, 4096, "bf16"),
    ("NT", True, 300, 1024, 512, "bf16"),     # ragged M, several tiles (64 x 128 tiles)
    ("NN", True, 77, 136, 320, "bf16"),       # ragged M and N (64 x 128 tiles)
    ("NT", True, 2048, 1024, 4096, "bf16"),   # k/v-shaped: 64 x 128 tiles fill the chip
    ("NT", True, 2048, 2048, 1024, "bf16"),   # 128 x 128 tiles
    ("NN", True, 2000, 2048, 512, "bf16"),    # 128 x 128 tiles, ragged M
    ("NT", False, 333, 256, 256, "bf16"),
    ("NN", False, 333, 256, 256, "bf16"),
    ("TN", False, 256, 256, 999, "bf16"),     # ragged K (token axis)
    ("NT", False, 100, 96, 80, "f32"),
    ("TN", False, 64, 48, 37, "f32"),
]


@pytest.mark.parametrize("layout,dense,M,N,K,dtype", GEMM_CASES)
def test_gemm_parity(layout, dense, M, N, K, dtype):
    ash = (M, K) if layout != "TN" else (K, M)
    bsh = (N, K) if layout == "NT" else (K, N)
    A = I.gaussian(ash, 1.0, dtype, 400, M, K)
    Bm = I.gaussian(bsh, 1.0, dtype, 401, N, K)
    C = torch.empty((M, N), dtype=tdtype(dtype), device=DEV)
    code_l = {"NT": B.POETX_GEMM_NT, "NN": B.POETX_GEMM_NN, "TN": B.POETX_GEMM_TN}[layout]
    B.poetx_gemm(code_l, dev(A, dtype), dev(Bm, dtype), C, M, N, K, dense=dense)
    a64, b64 = A.astype(np.float64), Bm.astype(np.float64)
    ref = {"NT": lambda: a64 @ b64.T, "NN": lambda: a64 @ b64, "TN": lambda: a64.T @ b64}[layout]()
    # bf16 output rounding (2^-9) on top of float32 accumulation
    assert rel_fro(host(C), ref) <= (4e-3 if dtype == "bf16" else 1e-6)


# bf16 token runs up to 4096 per split take the two-k-tiles-per-stage kernel,
# longer ones the four-stage one (4650: ragged, one split); 5000 x 1024 / 512
# splits the token axis in two ragged halves.
@pytest.mark.parametrize("T,d,b,dtype", [(2048, 4096, 256, "bf16"), (777, 512, 128, "bf16"), (50, 96, 32, "f32"),
                                         (0, 256, 64, "bf16"), (4650, 4096, 256, "bf16"), (5000, 1024, 512, "bf16")])
def test_block_grad_parity(T, d, b, dtype):
    A = I.gaussian((T, d), 1.0, dtype, 402, T, d)
    Bm = I.gaussian((T, d), 1.0, dtype, 403, T, d)
    dG = torch.full((d // b, b, b), 3.0, dtype=torch.float32, device=DEV)
    ws = B.workspace(B.poetx_block_grad_workspace_bytes(T, d, b, code(dtype)))
    B.poetx_block_grad(dev(A, dtype), dev(Bm, dtype), dG, T, d, b, ws)
    a64, b64 = A.astype(np.float64), Bm.astype(np.float64)
    ref = np.stack([a64[:, j * b:(j + 1) * b].T @ b64[:, j * b:(j + 1) * b] for j in range(d // b)])
    if T == 0:
        assert not dG.any()
    else:
        assert rel_fro(host(dG), ref) <= (1e-5 if dtype == "f32" else 1e-5)


@pytest.mark.parametrize("T,d,b,dtype", [(2048, 4096, 256, "bf16"), (2048, 1024, 256, "bf16"), (300, 1024, 512, "bf16"),
                                         (2100, 14336, 256, "bf16"), (4096, 4096, 512, "bf16"),
                                         (77, 192, 64, "bf16"), (33, 96, 32, "f32"), (129, 128, 16, "bf16")])
@pytest.mark.parametrize("transpose", [True, False])
def test_block_apply_parity(T, d, b, dtype, transpose):
    X = I.gaussian((T, d), 1.0, dtype, 404, T, d)
    G = I.gaussian((d // b, b, b), 0.1, dtype, 405, d, b)
    out = torch.empty((T, d), dtype=tdtype(dtype), device=DEV)
    B.poetx_block_apply(dev(X, dtype), dev(G, dtype), out, T, d, b, transpose_G=transpose)
    x64, g64 = X.astype(np.float64), G.astype(np.float64)
    ref = np.concatenate([x64[:, j * b:(j + 1) * b] @ (g64[j].T if transpose else g64[j]) for j in range(d // b)],
                         axis=1)
    assert rel_fro(host(out), ref) <= (4e-3 if dtype == "bf16" else 1e-6)
