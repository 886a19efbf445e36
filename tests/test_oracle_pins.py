"""Pins for the float64 oracle: each check ties the oracle to something other
than itself (a worked closed form, an identity of the mathematics, brute force,
finite differences, or an independent formulation of the same layer).

Sources: "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
Transformation" (SAI replication review: Summary, Weaknesses "Cayley
approximation", "Notation gaps", Reproducibility "Partial coverage") and the
agidaily.cc article (W_RP = R W0 P, merge-then-reinitialize).
"""
import os

import numpy as np
import pytest

from oracle import poet_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return rows


def _rand_q(rng, nblk, b, std):
    return rng.standard_normal((nblk, b * (b - 1) // 2)) * std


# ------------------------------------------------------------ skew storage
@pytest.mark.parametrize("name,b", [("skew_b3.txt", 3), ("skew_b4.txt", 4)])
def test_skew_layout_golden(name, b):
    rows = _read_rows(name)
    q = np.array(rows[0])
    Q_expect = np.array(rows[1:])
    Q = O.skew_from_params(q[None], b)[0]
    assert np.array_equal(Q, Q_expect)


def test_skew_exact_and_pack_adjoint():
    rng = np.random.default_rng(1)
    b = 7
    q = _rand_q(rng, 3, b, 1.0)
    Q = O.skew_from_params(q, b)
    assert np.array_equal(Q, -np.transpose(Q, (0, 2, 1)))
    assert np.all(np.diagonal(Q, axis1=1, axis2=2) == 0)
    # adjoint identity <unpack(q), M> = <q, pack(M)>
    M = rng.standard_normal((3, b, b))
    lhs = np.sum(Q * M)
    rhs = np.sum(q * O.params_grad_from_skew_grad(M))
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))
    # pack of a skew matrix gives twice its parameters
    assert np.allclose(O.params_grad_from_skew_grad(Q), 2 * q, rtol=0, atol=0)


# ------------------------------------------------------- Cayley-Neumann map
def test_cnp_b2_golden():
    for t, k, g00, g01, g10, g11 in _read_rows("cnp_b2.txt"):
        Q = np.array([[0.0, t], [-t, 0.0]])
        G = O.exact_cayley(Q) if k < 0 else O.neumann_cayley(Q, int(k))
        assert np.allclose(G, [[g00, g01], [g10, g11]], rtol=0, atol=1e-14), (t, k, G)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 6])
def test_cnp_b2_complex_closed_form(k):
    # Q = tJ with J^2 = -I behaves like z = i t:  G = Re f(it) I + Im f(it) J
    for t in (0.05, 0.3, 0.9, 1.7):
        z = 1j * t
        f = (1 + z) * sum(z ** i for i in range(k + 1))
        J = np.array([[0.0, 1.0], [-1.0, 0.0]])
        expect = f.real * np.eye(2) + f.imag * J
        G = O.neumann_cayley(t * J, k)
        assert np.allclose(G, expect, rtol=0, atol=1e-13)


@pytest.mark.parametrize("k", [1, 3, 4, 5])
def test_cnp_equals_exact_cayley_times_truncation(k):
    """(I+Q) sum_{i<=k} Q^i = (I+Q)(I-Q)^-1 (I - Q^{k+1}); since Q is normal and
    the Cayley transform orthogonal, ||R_exact - G_k||_2 = ||Q||_2^{k+1}."""
    rng = np.random.default_rng(10 + k)
    b = 8
    Q = O.skew_from_params(_rand_q(rng, 2, b, 0.2), b)
    G = O.neumann_cayley(Q, k)
    Rx = O.exact_cayley(Q)
    for j in range(2):
        Qk1 = np.linalg.matrix_power(Q[j], k + 1)
        assert np.allclose(G[j], Rx[j] @ (np.eye(b) - Qk1), rtol=0, atol=1e-13)
        nq = np.linalg.norm(Q[j], 2)
        assert abs(np.linalg.norm(Rx[j] - G[j], 2) - nq ** (k + 1)) < 1e-12
        # the exact Cayley transform is orthogonal
        assert np.allclose(Rx[j].T @ Rx[j], np.eye(b), atol=1e-13)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_cnp_singular_values(k):
    """Singular values of G_k are |1 - (i theta)^{k+1}| for the eigenvalues
    +-i theta of the skew block."""
    rng = np.random.default_rng(20 + k)
    b = 6
    Q = O.skew_from_params(_rand_q(rng, 1, b, 0.4), b)[0]
    lam = np.linalg.eigvals(Q)
    expect = np.sort(np.abs(1 - lam ** (k + 1)))
    sv = np.sort(np.linalg.svd(O.neumann_cayley(Q, k), compute_uv=False))
    assert np.allclose(sv, expect, rtol=0, atol=1e-12)


def test_cnp_first_order_is_identity_plus_2q():
    """The review corrects the paper's first-order claim to R ~ I + 2Q
    (Weaknesses, "Cayley approximation ..."): (G - I - 2 eps Q)/eps^2 -> 2 Q^2."""
    rng = np.random.default_rng(3)
    b = 5
    Q = O.skew_from_params(_rand_q(rng, 1, b, 1.0), b)[0]
    for eps in (1e-2, 1e-3):
        G = O.neumann_cayley(eps * Q, 3)
        second = (G - np.eye(b) - 2 * eps * Q) / eps ** 2
        assert np.allclose(second, 2 * Q @ Q, atol=10 * eps * np.linalg.norm(Q) ** 3)


def test_cnp_zero_is_identity():
    G = O.neumann_cayley(np.zeros((3, 4, 4)), 3)
    assert np.array_equal(G, np.broadcast_to(np.eye(4), (3, 4, 4)))


# ------------------------------------------------------- permutations, R, P
def test_orthogonal_from_blocks_is_conjugation():
    rng = np.random.default_rng(4)
    b, nblk = 3, 4
    G = rng.standard_normal((nblk, b, b))
    pi = rng.permutation(nblk * b)
    Pi = O.gather_matrix(pi)
    v = rng.standard_normal(nblk * b)
    assert np.array_equal(Pi @ v, v[pi])               # gather convention
    R = O.orthogonal_from_blocks(G, pi)
    assert np.allclose(R, Pi.T @ O.block_diag(G) @ Pi, rtol=0, atol=0)


def test_prepermute_brute_force():
    rng = np.random.default_rng(5)
    m, n = 6, 4
    W0 = rng.standard_normal((m, n))
    pi_R, pi_P = rng.permutation(m), rng.permutation(n)
    Wt = O.prepermute(W0, pi_R, pi_P)
    assert np.array_equal(Wt, O.gather_matrix(pi_R) @ W0 @ O.gather_matrix(pi_P).T)
    for i in range(m):
        for j in range(n):
            assert Wt[i, j] == W0[pi_R[i], pi_P[j]]


# -------------------------------------------------------------- forward
def _layer(rng, m=12, n=8, b=4, T=5, qstd=0.3):
    W0 = rng.standard_normal((m, n)) * 0.5
    q_R = _rand_q(rng, m // b, b, qstd)
    q_P = _rand_q(rng, n // b, b, qstd)
    x = rng.standard_normal((T, n))
    dy = rng.standard_normal((T, m))
    return W0, q_R, q_P, x, dy, rng.permutation(m), rng.permutation(n)


def test_q_zero_reduces_to_plain_linear():
    rng = np.random.default_rng(6)
    W0, q_R, q_P, x, dy, pi_R, pi_P = _layer(rng)
    y = O.forward(x, W0, 0 * q_R, 0 * q_P, pi_R, pi_P, 4, 3)
    assert np.allclose(y, x @ W0.T, rtol=0, atol=1e-14)


def test_input_centric_chain_matches_dense():
    """The matrix-free chain (review Summary: gather, batched blocks, the weight
    with two permutations absorbed, batched blocks, scatter) written with plain
    loops must equal the dense weight-centric R W0 P x."""
    rng = np.random.default_rng(7)
    m, n, b, T, k = 12, 8, 4, 5, 3
    W0, q_R, q_P, x, dy, pi_R, pi_P = _layer(rng, m, n, b, T)
    G_R = O.blocks_from_params(q_R, b, k)
    G_P = O.blocks_from_params(q_P, b, k)
    Wt = O.prepermute(W0, pi_R, pi_P)
    y = np.zeros((T, m))
    for t in range(T):
        a = np.array([x[t, pi_P[i]] for i in range(n)])
        h1 = np.zeros(n)
        for j in range(n // b):
            for r in range(b):
                h1[j * b + r] = sum(G_P[j, r, c] * a[j * b + c] for c in range(b))
        h2 = np.array([sum(Wt[i, c] * h1[c] for c in range(n)) for i in range(m)])
        z = np.zeros(m)
        for j in range(m // b):
            for r in range(b):
                z[j * b + r] = sum(G_R[j, r, c] * h2[j * b + c] for c in range(b))
        for i in range(m):
            y[t, pi_R[i]] = z[i]
    assert np.allclose(y, O.forward(x, W0, q_R, q_P, pi_R, pi_P, b, k), rtol=0, atol=1e-13)


def test_spectrum_preserved_under_exact_cayley():
    """Orthogonal equivalence keeps the singular values of W0 (review Summary)."""
    rng = np.random.default_rng(8)
    m, n, b = 12, 8, 4
    W0, q_R, q_P, *_rest, pi_R, pi_P = _layer(rng, m, n, b, qstd=0.8)
    G_R = O.blocks_from_params(q_R, b, 3, cayley="exact")
    G_P = O.blocks_from_params(q_P, b, 3, cayley="exact")
    W = O.effective_weight(W0, G_R, G_P, pi_R, pi_P)
    s0 = np.linalg.svd(W0, compute_uv=False)
    assert np.allclose(np.linalg.svd(W, compute_uv=False), s0, rtol=0, atol=1e-12)
    # with the truncated series the spectrum moves by at most the truncation
    q_small = 0.1
    _, q_R, q_P, *_ = _layer(np.random.default_rng(9), m, n, b, qstd=q_small)
    G_R = O.blocks_from_params(q_R, b, 3)
    G_P = O.blocks_from_params(q_P, b, 3)
    W = O.effective_weight(W0, G_R, G_P, pi_R, pi_P)
    eps = max(np.linalg.norm(Qj, 2) for Qj in
              list(O.skew_from_params(q_R, b)) + list(O.skew_from_params(q_P, b))) ** 4
    s = np.linalg.svd(W, compute_uv=False)
    assert np.all(np.abs(s - s0) <= ((1 + eps) ** 2 - 1) * s0 + 1e-13)


def test_forward_linear_in_x():
    rng = np.random.default_rng(11)
    W0, q_R, q_P, x, dy, pi_R, pi_P = _layer(rng)
    x2 = rng.standard_normal(x.shape)
    f = lambda v: O.forward(v, W0, q_R, q_P, pi_R, pi_P, 4, 3)
    assert np.allclose(f(2 * x - 3 * x2), 2 * f(x) - 3 * f(x2), atol=1e-12)


# -------------------------------------------------------------- backward
def _loss(dy, x, W0, q_R, q_P, pi_R, pi_P, b, k):
    return np.sum(dy * O.forward(x, W0, q_R, q_P, pi_R, pi_P, b, k))


@pytest.mark.parametrize("k", [3, 4, 2])
def test_backward_matches_finite_differences(k):
    rng = np.random.default_rng(12 + k)
    m, n, b, T = 12, 8, 4, 5
    W0, q_R, q_P, x, dy, pi_R, pi_P = _layer(rng, m, n, b, T)
    dx, dq_R, dq_P, _, _ = O.backward(dy, x, W0, q_R, q_P, pi_R, pi_P, b, k)
    h = 1e-6

    def fd(arr, setter):
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, mm = arr.copy(), arr.copy()
            p[idx] += h
            mm[idx] -= h
            g[idx] = (setter(p) - setter(mm)) / (2 * h)
        return g

    g_qR = fd(q_R, lambda v: _loss(dy, x, W0, v, q_P, pi_R, pi_P, b, k))
    g_qP = fd(q_P, lambda v: _loss(dy, x, W0, q_R, v, pi_R, pi_P, b, k))
    g_x = fd(x, lambda v: _loss(dy, v, W0, q_R, q_P, pi_R, pi_P, b, k))
    for got, ref in ((dq_R, g_qR), (dq_P, g_qP), (dx, g_x)):
        assert np.linalg.norm(got - ref) <= 1e-7 * np.linalg.norm(ref)


def test_cnp_vjp_matches_finite_differences():
    rng = np.random.default_rng(16)
    b = 5
    for k in (1, 3, 4):
        Q = O.skew_from_params(_rand_q(rng, 1, b, 0.5), b)[0]
        dG = rng.standard_normal((b, b))
        E = rng.standard_normal((b, b))       # unconstrained direction
        h = 1e-6
        fd = np.sum(dG * (O.neumann_cayley(Q + h * E, k) - O.neumann_cayley(Q - h * E, k))) / (2 * h)
        assert abs(np.sum(O.cnp_vjp(Q, dG, k) * E) - fd) < 1e-8 * max(1, abs(fd))


def test_backward_dx_is_dy_times_effective_weight():
    rng = np.random.default_rng(17)
    W0, q_R, q_P, x, dy, pi_R, pi_P = _layer(rng)
    dx, *_ = O.backward(dy, x, W0, q_R, q_P, pi_R, pi_P, 4, 3)
    W = O.effective_weight(W0, O.blocks_from_params(q_R, 4, 3), O.blocks_from_params(q_P, 4, 3),
                           pi_R, pi_P)
    assert np.allclose(dx, dy @ W, atol=1e-13)
    # adjoint (dot-product) test in x
    dlt = rng.standard_normal(x.shape)
    lhs = np.sum(dy * O.forward(dlt, W0, q_R, q_P, pi_R, pi_P, 4, 3))
    assert abs(lhs - np.sum(dx * dlt)) < 1e-12 * max(1, abs(lhs))


def test_zero_tokens_give_zero_block_gradients():
    rng = np.random.default_rng(18)
    W0, q_R, q_P, x, dy, pi_R, pi_P = _layer(rng, T=1)
    dx, dq_R, dq_P, dG_R, dG_P = O.backward(dy[:0], x[:0], W0, q_R, q_P, pi_R, pi_P, 4, 3)
    assert dx.shape == (0, 8) and not dG_R.any() and not dq_P.any()


# ----------------------------------------------------------------- merge
def test_merge_preserves_the_function():
    rng = np.random.default_rng(19)
    m, n, b, T, k = 12, 8, 4, 5, 3
    W0, q_R, q_P, x, dy, pi_R, pi_P = _layer(rng, m, n, b, T)
    Wt = O.prepermute(W0, pi_R, pi_P)
    pi_R2, pi_P2 = rng.permutation(m), rng.permutation(n)
    y_before = O.forward(x, W0, q_R, q_P, pi_R, pi_P, b, k)
    Wt2, q_R2, q_P2 = O.merge(Wt, q_R, q_P, pi_R, pi_P, pi_R2, pi_P2, b, k)
    assert not q_R2.any() and not q_P2.any()
    W0_after = O.gather_matrix(pi_R2).T @ Wt2 @ O.gather_matrix(pi_P2)
    y_after = O.forward(x, W0_after, q_R2, q_P2, pi_R2, pi_P2, b, k)
    assert np.allclose(y_after, y_before, rtol=0, atol=1e-13)
    # stored weight of the merged layer, element by element
    Weff = O.effective_weight(W0, O.blocks_from_params(q_R, b, k), O.blocks_from_params(q_P, b, k),
                              pi_R, pi_P)
    for i in range(m):
        for j in range(n):
            assert abs(Wt2[i, j] - Weff[pi_R2[i], pi_P2[j]]) < 1e-14


def test_merge_with_zero_q_and_same_perms_is_identity():
    rng = np.random.default_rng(20)
    W0, q_R, q_P, x, dy, pi_R, pi_P = _layer(rng)
    Wt = O.prepermute(W0, pi_R, pi_P)
    Wt2, _, _ = O.merge(Wt, 0 * q_R, 0 * q_P, pi_R, pi_P, pi_R, pi_P, 4, 3)
    assert np.array_equal(Wt2, Wt)


# ------------------------------------- outputs the oracle computes one by one
def _blocks(rng, nblk, b, k=3, std=0.3):
    return O.blocks_from_params(_rand_q(rng, nblk, b, std), b, k)


def _loss_g(dy, x, W0, G_R, G_P, pi_R, pi_P):
    return np.sum(dy * O.forward_from_blocks(x, W0, G_R, G_P, pi_R, pi_P))


def test_sampled_block_grads_match_finite_differences():
    # L = <dY, X P^T W0^T R^T> is linear in every entry of G_R and of G_P, so a
    # central difference is exact up to rounding.
    rng = np.random.default_rng(21)
    m, n, b, T = 12, 8, 4, 6
    W0, _, _, x, dy, pi_R, pi_P = _layer(rng, m, n, b, T)
    G_R, G_P = _blocks(rng, m // b, b), _blocks(rng, n // b, b)
    h = 1e-3
    for side, G, nblk in (("R", G_R, m // b), ("P", G_P, n // b)):
        entries = [(j, r, c) for j in range(nblk) for r in range(b) for c in range(b)]
        got = O.block_grad_entries(dy, x, W0, G_R, G_P, pi_R, pi_P, side, entries)
        whole = O.block_grad_blocks(dy, x, W0, G_R, G_P, pi_R, pi_P, side, list(range(nblk)))
        fd = np.empty(len(entries))
        for i, (j, r, c) in enumerate(entries):
            Gp, Gm = G.copy(), G.copy()
            Gp[j, r, c] += h
            Gm[j, r, c] -= h
            args_p = (Gp, G_P) if side == "R" else (G_R, Gp)
            args_m = (Gm, G_P) if side == "R" else (G_R, Gm)
            fd[i] = (_loss_g(dy, x, W0, *args_p, pi_R, pi_P) - _loss_g(dy, x, W0, *args_m, pi_R, pi_P)) / (2 * h)
        assert np.allclose(got, fd, rtol=0, atol=1e-9)
        assert np.allclose(whole.reshape(-1), fd, rtol=0, atol=1e-9)


def test_sampled_input_grad_rows_brute_force():
    # dx[t, i] = sum_o dy[t, o] * W_RP[o, i] with W_RP[o, i] = sum_{a, e} R[o, a] W0[a, e] P[e, i],
    # summed term by term from the block entries: R[pi_R[u], pi_R[v]] = G_R[u // b][u % b, v % b]
    # when u, v lie in the same block.
    rng = np.random.default_rng(22)
    m, n, b, T = 8, 6, 2, 3
    W0, _, _, x, dy, pi_R, pi_P = _layer(rng, m, n, b, T)
    G_R, G_P = _blocks(rng, m // b, b), _blocks(rng, n // b, b)

    def entry(G, pi, row, col):
        u, v = int(np.where(pi == row)[0][0]), int(np.where(pi == col)[0][0])
        return G[u // b][u % b, v % b] if u // b == v // b else 0.0

    W = np.zeros((m, n))
    for o in range(m):
        for i in range(n):
            W[o, i] = sum(entry(G_R, pi_R, o, a) * W0[a, e] * entry(G_P, pi_P, e, i)
                          for a in range(m) for e in range(n))
    rows = [2, 0]
    got = O.input_grad(dy[rows], W0, G_R, G_P, pi_R, pi_P)
    for t, row in enumerate(rows):
        for i in range(n):
            assert abs(got[t, i] - sum(dy[row, o] * W[o, i] for o in range(m))) < 1e-12
    y = O.forward_from_blocks(x[rows], W0, G_R, G_P, pi_R, pi_P)
    for t, row in enumerate(rows):
        for o in range(m):
            assert abs(y[t, o] - sum(W[o, i] * x[row, i] for i in range(n))) < 1e-12


def test_merge_entries_match_merged_function():
    # Folding the layer into the weight keeps y unchanged: with the merged stored
    # weight Wt', q = 0 and the new permutations, y = Pi_R'^T Wt' Pi_P' x.
    rng = np.random.default_rng(23)
    m, n, b, T, k = 12, 8, 4, 5, 3
    W0, q_R, q_P, x, _, pi_R, pi_P = _layer(rng, m, n, b, T)
    Wt = O.prepermute(W0, pi_R, pi_P)
    pi_R2, pi_P2 = rng.permutation(m), rng.permutation(n)
    G_R, G_P = O.blocks_from_params(q_R, b, k), O.blocks_from_params(q_P, b, k)
    entries = [(i, j) for i in range(m) for j in range(n)]
    Wt2 = O.merge_entries(Wt, G_R, G_P, pi_R, pi_P, pi_R2, pi_P2, entries).reshape(m, n)
    W_new = np.empty((m, n))
    W_new[np.ix_(pi_R2, pi_P2)] = Wt2
    y_before = O.forward(x, W0, q_R, q_P, pi_R, pi_P, b, k)
    assert np.allclose(x @ W_new.T, y_before, rtol=0, atol=1e-13)


# ------------------------------------------------------------ training step
# AdamW (Loshchilov and Hutter 2019; Adam's bias correction, Kingma and Ba 2015)
# at the rate lr * gamma, gamma = 0.5 being the POET learning-rate scaling
# (SAI replication review, Weaknesses, single-run 8B/13B remark).
_OPT = dict(lr=3e-3, gamma=0.5, beta1=0.9, beta2=0.999, eps=1e-8)


def test_adamw_constant_gradient_closed_form():
    # With a constant gradient the bias-corrected moments are g and g^2 at every
    # step, so each update is exactly lr gamma g / (|g| + eps).
    rng = np.random.default_rng(31)
    g = rng.standard_normal(50) * np.logspace(-4, 2, 50)
    q0 = rng.standard_normal(50)
    q, m, v = q0.copy(), np.zeros(50), np.zeros(50)
    for t in range(1, 8):
        q, m, v = O.adamw_step(q, g, m, v, t, **_OPT)
        want = q0 - t * _OPT["lr"] * _OPT["gamma"] * g / (np.abs(g) + _OPT["eps"])
        assert np.allclose(q, want, rtol=0, atol=1e-13)


def test_adamw_zero_gradient_is_pure_decay():
    # No gradient: the moments stay 0 and decoupled decay shrinks q
    # geometrically by (1 - lr gamma wd) per step.
    q0 = np.linspace(-2, 3, 11)
    q, m, v = q0.copy(), np.zeros(11), np.zeros(11)
    for t in range(1, 6):
        q, m, v = O.adamw_step(q, np.zeros(11), m, v, t, **_OPT, weight_decay=0.1)
    assert np.allclose(q, q0 * (1 - _OPT["lr"] * _OPT["gamma"] * 0.1) ** 5, rtol=1e-15, atol=0)
    assert not m.any() and not v.any()


def test_adamw_matches_library_optimizer():
    # torch.optim.AdamW in float64 on the CPU, at the scaled rate, over a random
    # gradient sequence with weight decay.
    import torch
    rng = np.random.default_rng(32)
    n, steps, wd = 40, 9, 0.05
    grads = rng.standard_normal((steps, n)) * rng.uniform(1e-3, 10, n)
    q0 = rng.standard_normal(n)
    p = torch.tensor(q0.copy(), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=_OPT["lr"] * _OPT["gamma"], betas=(_OPT["beta1"], _OPT["beta2"]),
                            eps=_OPT["eps"], weight_decay=wd)
    q, m, v = q0.copy(), np.zeros(n), np.zeros(n)
    for t in range(1, steps + 1):
        p.grad = torch.tensor(grads[t - 1], dtype=torch.float64)
        opt.step()
        q, m, v = O.adamw_step(q, grads[t - 1], m, v, t, **_OPT, weight_decay=wd)
    assert np.allclose(q, p.detach().numpy(), rtol=0, atol=1e-14)


def test_adamw_is_invariant_to_gradient_scale():
    rng = np.random.default_rng(33)
    grads = rng.standard_normal((6, 30))
    opt = dict(_OPT, eps=0.0)
    a = b = (rng.standard_normal(30), np.zeros(30), np.zeros(30))
    for t in range(1, 7):
        a = O.adamw_step(*a[:1], grads[t - 1], *a[1:], t, **opt)
        b = O.adamw_step(*b[:1], 1e3 * grads[t - 1], *b[1:], t, **opt)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-13)


def _train_case(rng, steps, m=12, n=8, b=4, T=5):
    W0, q_R, q_P, _, _, pi_R, pi_P = _layer(rng, m, n, b, T)
    xs = rng.standard_normal((steps, T, n))
    dys = rng.standard_normal((steps, T, m))
    perms = [(rng.permutation(m), rng.permutation(n)) for _ in range(4)]
    return W0, q_R, q_P, pi_R, pi_P, xs, dys, perms


def test_train_step_decreases_the_loss_to_first_order():
    # One step at a tiny rate changes L = <dY, Y> by <dq, delta q> to first
    # order: the update goes against the gradient of L with respect to q, at the
    # scaled rate.
    rng = np.random.default_rng(34)
    b, k = 4, 3
    W0, q_R, q_P, pi_R, pi_P, xs, dys, _ = _train_case(rng, 1)
    opt = dict(_OPT, lr=1e-7)
    _, q_R1, q_P1, _, _ = O.train_steps(xs, dys, W0, q_R, q_P, pi_R, pi_P, b, k, opt, 400, iter(()))
    L = lambda qr, qp: np.sum(dys[0] * O.forward(xs[0], W0, qr, qp, pi_R, pi_P, b, k))
    _, dq_R, dq_P, _, _ = O.backward(dys[0], xs[0], W0, q_R, q_P, pi_R, pi_P, b, k)
    eta = opt["lr"] * opt["gamma"]
    want = -eta * (np.sum(dq_R ** 2 / (np.abs(dq_R) + opt["eps"])) + np.sum(dq_P ** 2 / (np.abs(dq_P) + opt["eps"])))
    got = L(q_R1, q_P1) - L(q_R, q_P)
    assert want < 0 and abs(got - want) < 1e-4 * abs(want)


def test_train_merge_keeps_the_function():
    # At the merge step the layer's function is the one the last update left:
    # the merged weight with q = 0 and the new permutations computes what the
    # unmerged weight with the updated q computes.
    rng = np.random.default_rng(35)
    b, k, M = 4, 3, 3
    W0, q_R, q_P, pi_R, pi_P, xs, dys, perms = _train_case(rng, M)
    Wt_a, qR_a, qP_a, piR_a, piP_a = O.train_steps(xs, dys, W0, q_R, q_P, pi_R, pi_P, b, k, _OPT, M + 1, iter(()))
    Wt_b, qR_b, qP_b, piR_b, piP_b = O.train_steps(xs, dys, W0, q_R, q_P, pi_R, pi_P, b, k, _OPT, M, iter(perms))
    assert not qR_b.any() and not qP_b.any()
    assert np.array_equal(piR_b, perms[0][0]) and np.array_equal(piP_b, perms[0][1])
    assert np.array_equal(piR_a, pi_R) and not np.allclose(qR_a, q_R)
    x = rng.standard_normal((7, W0.shape[1]))
    W0_a = Wt_a[np.argsort(piR_a)][:, np.argsort(piP_a)]
    W0_b = Wt_b[np.argsort(piR_b)][:, np.argsort(piP_b)]
    assert np.allclose(O.forward(x, W0_a, qR_a, qP_a, piR_a, piP_a, b, k), x @ W0_b.T, rtol=0, atol=1e-12)


def test_train_after_merge_starts_afresh():
    # After a merge nothing of the previous segment survives but the weight: two
    # segments of M steps equal one segment of M steps followed by a new run of
    # M steps from the merged state (moments and count reset with q).
    rng = np.random.default_rng(36)
    b, k, M = 4, 3, 3
    W0, q_R, q_P, pi_R, pi_P, xs, dys, perms = _train_case(rng, 2 * M)
    full = O.train_steps(xs, dys, W0, q_R, q_P, pi_R, pi_P, b, k, _OPT, M, iter(perms))
    Wt1, qR1, qP1, piR1, piP1 = O.train_steps(xs[:M], dys[:M], W0, q_R, q_P, pi_R, pi_P, b, k, _OPT, M,
                                              iter(perms[:1]))
    W0_1 = Wt1[np.argsort(piR1)][:, np.argsort(piP1)]
    second = O.train_steps(xs[M:], dys[M:], W0_1, qR1, qP1, piR1, piP1, b, k, _OPT, M, iter(perms[1:]))
    for a, c in zip(full, second):
        assert np.allclose(a, c, rtol=0, atol=1e-12)


# ------------------------------------------------------- POET-XQ storage
def test_quantize_rows_hand_example():
    # row 0: amax 1.27 -> scale 0.01 (float32); 0.5 / 0.01 = 50, -0.333 / 0.01 = -33.3 -> -33
    # row 1: all zeros -> scale 0, codes 0;  row 2: a single nonzero maps to +-127
    W = np.array([[1.27, 0.5, -0.333, 0.0], [0.0, 0.0, 0.0, 0.0], [0.0, -3.0, 0.0, 0.0]], dtype=np.float32)
    q, s = O.quantize_rows_int8(W)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert q[0].tolist() == [127, 50, -33, 0]
    assert s[1] == 0 and q[1].tolist() == [0, 0, 0, 0]
    assert q[2].tolist() == [0, -127, 0, 0] and s[2] == np.float32(3.0) / np.float32(127.0)


def test_quantize_rows_is_nearest_grid_point_by_brute_force():
    rng = np.random.default_rng(41)
    W = (rng.standard_normal((6, 40)) * rng.uniform(0.01, 3.0, (6, 1))).astype(np.float32)
    q, s = O.quantize_rows_int8(W)
    ks = np.arange(-127, 128, dtype=np.float64)
    for i in range(W.shape[0]):
        grid = ks * np.float64(s[i])
        for j in range(W.shape[1]):
            d = np.abs(W[i, j] - grid)
            best = d.min()
            # the code is a nearest grid point (a float32 tie may go either way)
            assert abs(W[i, j] - q[i, j] * np.float64(s[i])) <= best + 1e-6 * s[i]
        assert np.abs(q[i]).max() == 127   # the largest entry sits on the end of the grid
    err = np.abs(O.dequantize_rows(q, s) - W)
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-5))


def test_quantize_rows_round_trips_values_on_the_grid():
    rng = np.random.default_rng(42)
    codes = rng.integers(-127, 128, (5, 33)).astype(np.int8)
    codes[:, 0] = 127
    scale = rng.uniform(0.001, 0.1, 5).astype(np.float32)
    # the scale is recomputed from the row maximum: amax = 127 * s exactly in float32 when
    # 127 * s is representable; take s = amax / 127 as the quantizer does
    amax = (np.float32(127.0) * scale).astype(np.float32)
    s2 = (amax / np.float32(127.0)).astype(np.float32)
    W = (codes.astype(np.float32) * s2[:, None]).astype(np.float32)
    q, s = O.quantize_rows_int8(W)
    assert np.array_equal(s, s2)
    assert np.array_equal(q, codes)
