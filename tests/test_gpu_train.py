"""GPU parity of the training step around the layer: the AdamW update of the
compact parameters at the POET-scaled rate, the optimizer reset, and a short
training loop (forward, backward, update, merge every few steps) against the
float64 oracle.  Float32 throughout: relative Frobenius error 1e-5."""
import numpy as np
import pytest
import torch

from oracle import poet_oracle as O
from orthogonal_equivalence_poet_amd import binding as B
from orthogonal_equivalence_poet_amd import inputs as I
from tests.gpu_helpers import DEV, cnp_bwd, cnp_fwd, dev, dev_i32, host, rel_fro

pytestmark = pytest.mark.gpu

TOL = 1e-5
OPT = dict(lr=2e-3, gamma=0.5, beta1=0.9, beta2=0.999, eps=1e-8)


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield
    torch.cuda.synchronize()


def _state(count, seed, q_std=1e-2):
    q = I.gaussian((count,), q_std, "f32", 95, seed, 0)
    grads = [I.gaussian((count,), 1.0, "f32", 95, seed, 1 + s) * np.float32(10.0 ** (s % 3 - 1)) for s in range(5)]
    return q, grads


def _run_gpu(q, grads, count, wd, offset=0, start_step=1):
    # rows of a multiple of 4 floats: offset 0 keeps all four arrays 16-byte
    # aligned (the vector path), offset 1 takes them off it (the scalar path)
    buf = torch.zeros((4, (count + offset + 7) // 4 * 4), dtype=torch.float32, device=DEV)
    qd, gd, md, vd = (buf[i, offset:offset + count] for i in range(4))
    qd.copy_(torch.from_numpy(q))
    p = B.adamw_params(**OPT, weight_decay=wd)
    for s, g in enumerate(grads):
        gd.copy_(torch.from_numpy(g))
        B.poetx_adamw_step(qd, gd, md, vd, count, start_step + s, p)
    return host(qd), host(md), host(vd), buf


def _run_oracle(q, grads, wd):
    m = v = np.zeros(q.shape)
    qo = q.astype(np.float64)
    for s, g in enumerate(grads):
        qo, m, v = O.adamw_step(qo, g, m, v, s + 1, **OPT, weight_decay=wd)
    return qo, m, v


@pytest.mark.parametrize("count", [1, 3, 4, 5, 1000, 1021, 4096 + 7, 262144 + 3])
@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_adamw_step_parity(count, offset, wd):
    q, grads = _state(count, count)
    qg, mg, vg, buf = _run_gpu(q, grads, count, wd, offset)
    qo, mo, vo = _run_oracle(q, grads, wd)
    assert rel_fro(qg, qo) < TOL and rel_fro(mg, mo) < TOL and rel_fro(vg, vo) < TOL
    # the change of q, not only q, is held to the bar
    assert rel_fro(qg - q, qo - q) < TOL
    # nothing outside the arrays is touched
    pad = host(buf)
    assert not pad[:, :offset].any() and not pad[:, offset + count:].any()


def test_adamw_constant_gradient_closed_form():
    # Constant gradient: the bias-corrected moments are g and g^2 at every step,
    # so each update is lr gamma g / (|g| + eps) (lr gamma sign(g) for |g| >> eps)
    # and from q = 0, q_t = -t lr gamma g / (|g| + eps).
    count = 4099
    g = I.gaussian((count,), 1.0, "f32", 96, 1)
    qg, _, _, _ = _run_gpu(np.zeros(count, np.float32), [g] * 4, count, 0.0)
    g64 = g.astype(np.float64)
    want = -4 * OPT["lr"] * OPT["gamma"] * g64 / (np.abs(g64) + OPT["eps"])
    assert np.max(np.abs(qg - want)) < 1e-6 * np.max(np.abs(want))


def test_adamw_zero_count_and_reset():
    B.poetx_adamw_step(None, None, None, None, 0, 1, B.adamw_params(1e-3))
    count = 1001
    m = torch.randn(count + 3, device=DEV)
    v = torch.randn(count + 3, device=DEV)
    B.poetx_adamw_reset(m, v, count)
    mh, vh = host(m), host(v)
    assert not mh[:count].any() and not vh[:count].any()
    assert np.all(mh[count:] != 0) and np.all(vh[count:] != 0)


def test_adamw_full_layer_parameter_count():
    # Every q of a Llama-8B-shaped layer (seven linears, b = 256) in one call.
    count = sum((s.nblk_R + s.nblk_P) * s.ntri for s in I.llama8b_layer())
    q, grads = _state(count, 7)
    grads = grads[:2]
    qg, mg, vg, _ = _run_gpu(q, grads, count, 0.0)
    qo, mo, vo = _run_oracle(q, grads, 0.0)
    assert rel_fro(qg - q, qo - q) < TOL and rel_fro(mg, mo) < TOL and rel_fro(vg, vo) < TOL


# ----------------------------------------------------------- training loop
def _train_gpu(spec, inp, xs, dys, perms, merge_every):
    s = spec
    d = B.desc(s.T, s.m, s.n, s.b, s.k, B.POETX_F32, B.POETX_FAST)
    Wt = torch.empty((s.m, s.n), dtype=torch.float32, device=DEV)
    pi_R, pi_P = dev_i32(inp["pi_R"]), dev_i32(inp["pi_P"])
    B.poetx_prepermute(dev(inp["W0"]), Wt, s.m, s.n, pi_R, pi_P)
    q_R, q_P = dev(inp["q_R"]), dev(inp["q_P"])
    st = {name: torch.zeros_like(t) for name, t in (("mR", q_R), ("vR", q_R), ("mP", q_P), ("vP", q_P))}
    saved = B.workspace(B.poetx_linear_saved_bytes(d))
    ws_f = B.workspace(B.poetx_linear_fwd_workspace_bytes(d))
    ws_b = B.workspace(B.poetx_linear_bwd_workspace_bytes(d))
    ws_m = B.workspace(B.poetx_merge_workspace_bytes(d))
    p = B.adamw_params(**OPT)
    y = torch.empty((s.T, s.m), dtype=torch.float32, device=DEV)
    dx = torch.empty((s.T, s.n), dtype=torch.float32, device=DEV)
    dG_R = torch.empty((s.nblk_R, s.b, s.b), dtype=torch.float32, device=DEV)
    dG_P = torch.empty((s.nblk_P, s.b, s.b), dtype=torch.float32, device=DEV)
    t = 0
    new = iter(perms)
    for x_np, dy_np in zip(xs, dys):
        x, dy = dev(x_np), dev(dy_np)
        G_R = cnp_fwd(q_R, s.nblk_R, s.b, s.k, "f32")
        G_P = cnp_fwd(q_P, s.nblk_P, s.b, s.k, "f32")
        B.poetx_linear_fwd(d, x, Wt, G_R, G_P, pi_R, pi_P, y, saved, ws_f)
        B.poetx_linear_bwd(d, dy, x, Wt, G_R, G_P, pi_R, pi_P, saved, dx, dG_R, dG_P, ws_b)
        dq_R = cnp_bwd(q_R, dG_R, s.nblk_R, s.b, s.k, "f32")
        dq_P = cnp_bwd(q_P, dG_P, s.nblk_P, s.b, s.k, "f32")
        t += 1
        B.poetx_adamw_step(q_R, dq_R, st["mR"], st["vR"], q_R.numel(), t, p)
        B.poetx_adamw_step(q_P, dq_P, st["mP"], st["vP"], q_P.numel(), t, p)
        if t == merge_every:
            pr, pp = next(new)
            pr, pp = dev_i32(pr), dev_i32(pp)
            B.poetx_merge(d, Wt, q_R, q_P, pi_R, pi_P, pr, pp, ws_m)
            B.poetx_adamw_reset(st["mR"], st["vR"], q_R.numel())
            B.poetx_adamw_reset(st["mP"], st["vP"], q_P.numel())
            pi_R, pi_P, t = pr, pp, 0
    return host(Wt), host(q_R), host(q_P), host(pi_R).astype(np.int64), host(pi_P).astype(np.int64)


@pytest.mark.parametrize("m,n,b,T,steps,merge_every", [(64, 48, 16, 40, 7, 3), (256, 128, 64, 100, 5, 2)])
def test_training_loop_parity(m, n, b, T, steps, merge_every):
    spec = I.LinearSpec("train", m=m, n=n, b=b, k=3, T=T, dtype="f32", q_std=0.0, key=(12, m, n))
    inp = I.make_linear_inputs(spec, with_grad=False)
    xs = [I.gaussian((T, n), 1.0, "f32", 12, m, n, 100 + i) for i in range(steps)]
    dys = [I.gaussian((T, m), 1.0, "f32", 12, m, n, 200 + i) for i in range(steps)]
    perms = [(I.permutation(m, 12, m, 300 + i), I.permutation(n, 12, n, 400 + i)) for i in range(steps)]
    got = _train_gpu(spec, inp, xs, dys, perms, merge_every)
    want = O.train_steps(xs, dys, inp["W0"], inp["q_R"], inp["q_P"], inp["pi_R"], inp["pi_P"], b, 3, OPT,
                         merge_every, iter(perms))
    assert np.array_equal(got[3], want[3]) and np.array_equal(got[4], want[4])
    assert rel_fro(got[0], want[0]) < TOL
    # q has moved since the last merge (steps % merge_every updates)
    assert np.abs(want[1]).max() > 0
    assert rel_fro(got[1], want[1]) < TOL and rel_fro(got[2], want[2]) < TOL


# ------------------------------------------------ a layer's linears in one batch
@pytest.mark.parametrize("dtype,variant", [("f32", B.POETX_FAST), ("bf16", B.POETX_MEM)])
def test_layer_linears_share_one_cayley_neumann_batch(dtype, variant):
    """Several linears of one layer (different shapes, same b and k) run their
    Cayley-Neumann forward and backward as one flat batch of blocks, each
    linear taking views into the flat q, G, dG and dq; every linear's outputs
    match the oracle run on it alone."""
    b, k, T = 64, 3, 80
    shapes = [(256, 128), (64, 256), (192, 192)]
    specs = [I.LinearSpec("layer", m=m, n=n, b=b, k=k, T=T, dtype=dtype, q_std=0.02, key=(14, i, m))
             for i, (m, n) in enumerate(shapes)]
    inps = [I.make_linear_inputs(sp) for sp in specs]
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    code = B.POETX_F32 if dtype == "f32" else B.POETX_BF16
    nbs = [sp.nblk_R + sp.nblk_P for sp in specs]
    nall = sum(nbs)
    q_all = torch.cat([torch.cat([dev(inp["q_R"]), dev(inp["q_P"])]) for inp in inps]).contiguous()
    G_all = torch.empty((nall, b, b), dtype=td, device=DEV)
    dG_all = torch.empty((nall, b, b), dtype=torch.float32, device=DEV)
    dq_all = torch.empty_like(q_all)
    cnp_saved = B.workspace(B.poetx_cnp_saved_bytes(nall, b, k, code))
    cnp_ws = B.workspace(max(B.poetx_cnp_fwd_workspace_bytes(nall, b, k, code),
                             B.poetx_cnp_bwd_workspace_bytes(nall, b, k, code)))
    st = []
    o = 0
    for sp, inp, nb in zip(specs, inps, nbs):
        d = B.desc(T, sp.m, sp.n, b, k, code, variant)
        S = {"d": d, "sp": sp, "x": dev(inp["x"], dtype), "dy": dev(inp["dy"], dtype),
             "pi_R": dev_i32(inp["pi_R"]), "pi_P": dev_i32(inp["pi_P"]),
             "G_R": G_all[o:o + sp.nblk_R], "G_P": G_all[o + sp.nblk_R:o + nb],
             "dG_R": dG_all[o:o + sp.nblk_R], "dG_P": dG_all[o + sp.nblk_R:o + nb],
             "dq": dq_all[o:o + nb],
             "y": torch.empty((T, sp.m), dtype=td, device=DEV), "dx": torch.empty((T, sp.n), dtype=td, device=DEV),
             "saved": B.workspace(B.poetx_linear_saved_bytes(d)),
             "ws": B.workspace(max(B.poetx_linear_fwd_workspace_bytes(d), B.poetx_linear_bwd_workspace_bytes(d)))}
        S["Wt"] = torch.empty((sp.m, sp.n), dtype=td, device=DEV)
        B.poetx_prepermute(dev(inp["W0"], dtype), S["Wt"], sp.m, sp.n, S["pi_R"], S["pi_P"])
        st.append(S)
        o += nb
    B.poetx_cnp_fwd_save(q_all, nall, b, k, G_all, cnp_saved, cnp_ws)
    for S in st:
        B.poetx_linear_fwd(S["d"], S["x"], S["Wt"], S["G_R"], S["G_P"], S["pi_R"], S["pi_P"], S["y"], S["saved"],
                           S["ws"])
    for S in reversed(st):
        B.poetx_linear_bwd(S["d"], S["dy"], S["x"], S["Wt"], S["G_R"], S["G_P"], S["pi_R"], S["pi_P"], S["saved"],
                           S["dx"], S["dG_R"], S["dG_P"], S["ws"])
    B.poetx_cnp_bwd_saved(q_all, dG_all, nall, b, k, dq_all, code, cnp_saved, cnp_ws)
    torch.cuda.synchronize()
    tolr = TOL if dtype == "f32" else 1.5e-2
    for S, inp in zip(st, inps):
        sp = S["sp"]
        args = (inp["W0"], inp["q_R"], inp["q_P"], inp["pi_R"], inp["pi_P"], b, k)
        y = O.forward(inp["x"], *args)
        dx, dq_R, dq_P, _, _ = O.backward(inp["dy"], inp["x"], *args)
        dq = host(S["dq"])
        assert rel_fro(host(S["y"]), y) < tolr and rel_fro(host(S["dx"]), dx) < tolr
        assert rel_fro(dq[:sp.nblk_R], dq_R) < tolr and rel_fro(dq[sp.nblk_R:], dq_P) < tolr
