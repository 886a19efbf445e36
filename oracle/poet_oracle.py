"""Plain float64 CPU oracle for the POET-X linear layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run this module; the library path
never does.  It shares no code with the HIP kernels: it imports numpy only.

What it computes (sources are the pages' titles and sections):
  * "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
    Transformation", SAI replication review, Summary: every weight is trained
    through an orthogonal equivalence W_RP = R W0 P with W0 frozen; R and P are
    block-diagonal orthogonal matrices in a random permuted basis, built by the
    Cayley-Neumann parameterization (CNP) from a skew-symmetric Q stored as its
    upper triangle; two of the four permutations are absorbed into W0.
  * same review, Weaknesses ("Cayley approximation ..."): the first-order
    expansion of the Cayley map is I + 2Q, which fixes R = (I+Q)(I-Q)^-1.
  * same review, Reproducibility ("Partial coverage ..."): the fused kernel
    follows the paper's Eq. 8/9 with k = 3 and stores b(b-1)/2 elements per block.
  * agidaily.cc article (the W_RP = R W0 P formula and merge-then-reinitialize).

Everything is the dense definition written out: dense R and P are formed, the
layer is y_t = R W0 P x_t, and gradients are those of L = <dY, Y>.  Readings
taken where the pages are silent (all listed in the design notes):
  * Q[r, c] = q[idx(r, c)] for r < c in row-major order of the strict upper
    triangle, Q[c, r] = -Q[r, c], zero diagonal;
  * k is the highest power kept: G = (I + Q) * sum_{i=0..k} Q^i;
  * a permutation pi acts by gather, (Pi v)[i] = v[pi[i]], i.e. Pi[i, pi[i]] = 1,
    and R = Pi_R^T D_R Pi_R with D_R = blockdiag(G_R,0, G_R,1, ...);
  * the absorbed permutations are the two next to W0:  Wt = Pi_R W0 Pi_P^T;
  * merge folds R W0 P into the weight, resamples both permutations and sets
    q to zero;
  * the quantized variant (the review's POET-XQ, Summary and Strengths: the
    checkpointed variant never keeps a dequantized weight, and the comparison
    is with 8-bit methods) stores the pre-permuted weight as symmetric int8
    per output row; the pages give no format, this is the plainest 8-bit one.

All functions take and return numpy float64 arrays (float32 inputs are widened
losslessly); permutations are integer arrays.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "triangle_pairs", "skew_from_params", "params_grad_from_skew_grad",
    "neumann_cayley", "exact_cayley", "block_diag", "gather_matrix",
    "orthogonal_from_blocks", "prepermute", "blocks_from_params",
    "forward", "forward_from_blocks", "backward", "backward_from_blocks",
    "cnp_vjp", "merge", "effective_weight",
    "input_grad", "block_grad_entries", "block_grad_blocks", "merge_entries",
    "adamw_step", "train_steps", "quantize_rows_int8", "dequantize_rows",
]


# --------------------------------------------------------------- skew storage
def triangle_pairs(b: int):
    """Storage order of the b(b-1)/2 upper-triangle parameters: row-major over
    the strict upper triangle, i.e. (0,1), (0,2), ..., (0,b-1), (1,2), ..."""
    return [(r, c) for r in range(b) for c in range(r + 1, b)]


def skew_from_params(q: np.ndarray, b: int) -> np.ndarray:
    """Compact parameters [nblk, b(b-1)/2] -> skew blocks Q [nblk, b, b].

    Compact skew-symmetric storage (review Summary; b(b-1)/2 elements per block
    in the Reproducibility section)."""
    q = np.asarray(q, dtype=np.float64)
    if q.ndim == 1:
        q = q[None, :]
    nblk = q.shape[0]
    assert q.shape[1] == b * (b - 1) // 2
    Q = np.zeros((nblk, b, b), dtype=np.float64)
    for i, (r, c) in enumerate(triangle_pairs(b)):
        Q[:, r, c] = q[:, i]
        Q[:, c, r] = -q[:, i]
    return Q


def params_grad_from_skew_grad(dQ: np.ndarray) -> np.ndarray:
    """Adjoint of skew_from_params: dL/dq[idx(r,c)] = dL/dQ[r,c] - dL/dQ[c,r]."""
    dQ = np.asarray(dQ, dtype=np.float64)
    if dQ.ndim == 2:
        dQ = dQ[None]
    b = dQ.shape[1]
    pairs = triangle_pairs(b)
    dq = np.zeros((dQ.shape[0], len(pairs)), dtype=np.float64)
    for i, (r, c) in enumerate(pairs):
        dq[:, i] = dQ[:, r, c] - dQ[:, c, r]
    return dq


# ------------------------------------------------------ Cayley-Neumann blocks
def neumann_cayley(Q: np.ndarray, k: int) -> np.ndarray:
    """Truncated Cayley map G = (I + Q) * sum_{i=0..k} Q^i, with explicit powers.

    The Cayley transform (I+Q)(I-Q)^-1 with (I-Q)^-1 replaced by its Neumann
    series cut after Q^k (review Summary, "Cayley-Neumann orthogonalization";
    k = 3 in the Reproducibility section).  Works on [b, b] or [nblk, b, b]."""
    Q = np.asarray(Q, dtype=np.float64)
    single = Q.ndim == 2
    if single:
        Q = Q[None]
    b = Q.shape[-1]
    eye = np.eye(b)
    out = np.empty_like(Q)
    for j in range(Q.shape[0]):
        series = np.zeros((b, b))
        for i in range(k + 1):
            series = series + np.linalg.matrix_power(Q[j], i)
        out[j] = (eye + Q[j]) @ series
    return out[0] if single else out


def exact_cayley(Q: np.ndarray) -> np.ndarray:
    """Exact Cayley transform (I + Q)(I - Q)^-1 by a linear solve (pins only)."""
    Q = np.asarray(Q, dtype=np.float64)
    single = Q.ndim == 2
    if single:
        Q = Q[None]
    b = Q.shape[-1]
    eye = np.eye(b)
    # X (I - Q) = (I + Q)  <=>  (I - Q)^T X^T = (I + Q)^T
    out = np.stack([np.linalg.solve((eye - Qj).T, (eye + Qj).T).T for Qj in Q])
    return out[0] if single else out


def blocks_from_params(q: np.ndarray, b: int, k: int, cayley: str = "neumann") -> np.ndarray:
    Q = skew_from_params(q, b)
    if cayley == "exact":
        return exact_cayley(Q)
    return neumann_cayley(Q, k)


# ------------------------------------------------------- dense R, P and Wt
def block_diag(G: np.ndarray) -> np.ndarray:
    """D = diag(G_0, G_1, ...) as a dense matrix."""
    G = np.asarray(G, dtype=np.float64)
    nblk, b, _ = G.shape
    D = np.zeros((nblk * b, nblk * b))
    for j in range(nblk):
        D[j * b:(j + 1) * b, j * b:(j + 1) * b] = G[j]
    return D


def gather_matrix(pi: np.ndarray) -> np.ndarray:
    """Permutation matrix Pi with Pi[i, pi[i]] = 1, so (Pi v)[i] = v[pi[i]]."""
    pi = np.asarray(pi, dtype=np.int64)
    d = pi.shape[0]
    Pm = np.zeros((d, d))
    Pm[np.arange(d), pi] = 1.0
    return Pm


def orthogonal_from_blocks(G: np.ndarray, pi: np.ndarray) -> np.ndarray:
    """R = Pi^T D Pi: block-diagonal in the basis permuted by pi.

    Entry-wise this is R[pi[i], pi[j]] = D[i, j]; the tests check it against
    the product with explicit permutation matrices."""
    D = block_diag(G)
    pi = np.asarray(pi, dtype=np.int64)
    R = np.empty_like(D)
    R[np.ix_(pi, pi)] = D
    return R


def prepermute(W0: np.ndarray, pi_R: np.ndarray, pi_P: np.ndarray) -> np.ndarray:
    """Weight with the two inner permutations absorbed: Wt = Pi_R W0 Pi_P^T,
    i.e. Wt[i, j] = W0[pi_R[i], pi_P[j]] (review Summary, "permutation reduction")."""
    W0 = np.asarray(W0, dtype=np.float64)
    return W0[np.asarray(pi_R, dtype=np.int64)][:, np.asarray(pi_P, dtype=np.int64)]


def effective_weight(W0, G_R, G_P, pi_R, pi_P) -> np.ndarray:
    """W_RP = R W0 P (dense)."""
    R = orthogonal_from_blocks(G_R, pi_R)
    P = orthogonal_from_blocks(G_P, pi_P)
    return R @ np.asarray(W0, dtype=np.float64) @ P


# ------------------------------------------------------------- the layer
def forward_from_blocks(x, W0, G_R, G_P, pi_R, pi_P) -> np.ndarray:
    """Y = X P^T W0^T R^T, i.e. y_t = R W0 P x_t for every token row x_t."""
    R = orthogonal_from_blocks(G_R, pi_R)
    P = orthogonal_from_blocks(G_P, pi_P)
    x = np.asarray(x, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    return x @ P.T @ W0.T @ R.T


def forward(x, W0, q_R, q_P, pi_R, pi_P, b: int, k: int, cayley: str = "neumann"):
    G_R = blocks_from_params(q_R, b, k, cayley)
    G_P = blocks_from_params(q_P, b, k, cayley)
    return forward_from_blocks(x, W0, G_R, G_P, pi_R, pi_P)


def _diag_blocks(M: np.ndarray, b: int) -> np.ndarray:
    nblk = M.shape[0] // b
    return np.stack([M[j * b:(j + 1) * b, j * b:(j + 1) * b] for j in range(nblk)])


def backward_from_blocks(dy, x, W0, G_R, G_P, pi_R, pi_P):
    """Gradients of L = <dY, Y> for Y = X P^T W0^T R^T.  W0 is frozen: no dW0.

    Returns (dx, dG_R, dG_P) with
      dX = dY R W0 P,
      dR = dY^T X P^T W0^T,   dP = W0^T R^T dY^T X,
      dD_R = Pi_R dR Pi_R^T and dG_R,j its j-th diagonal block (P likewise)."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    b = G_R.shape[-1]
    R = orthogonal_from_blocks(G_R, pi_R)
    P = orthogonal_from_blocks(G_P, pi_P)
    dx = dy @ R @ W0 @ P
    dR = (dy.T @ x) @ P.T @ W0.T
    dP = (W0.T @ R.T) @ (dy.T @ x)
    PiR = np.asarray(pi_R, dtype=np.int64)
    PiP = np.asarray(pi_P, dtype=np.int64)
    dD_R = dR[np.ix_(PiR, PiR)]          # = Pi_R dR Pi_R^T
    dD_P = dP[np.ix_(PiP, PiP)]
    return dx, _diag_blocks(dD_R, b), _diag_blocks(dD_P, b)


def _poly_cnp(X: np.ndarray, k: int) -> np.ndarray:
    """f(X) = (I + X) sum_{i=0..k} X^i for a square (possibly 2b x 2b) matrix."""
    eye = np.eye(X.shape[0])
    series = np.zeros_like(X)
    for i in range(k + 1):
        series = series + np.linalg.matrix_power(X, i)
    return (eye + X) @ series


def cnp_vjp(Q: np.ndarray, dG: np.ndarray, k: int) -> np.ndarray:
    """Adjoint of the truncated Cayley map: dQ = L_f(Q^T, dG).

    The Frechet derivative of a polynomial f at A in direction E is the
    upper-right block of f([[A, E], [0, A]]) (block-triangular formula,
    Higham, Functions of Matrices, 2008, sec. 3.2); for a real polynomial the
    Frobenius adjoint of L_f(A, .) is L_f(A^T, .)."""
    Q = np.asarray(Q, dtype=np.float64)
    dG = np.asarray(dG, dtype=np.float64)
    single = Q.ndim == 2
    if single:
        Q, dG = Q[None], dG[None]
    b = Q.shape[-1]
    out = np.empty_like(Q)
    for j in range(Q.shape[0]):
        big = np.zeros((2 * b, 2 * b))
        big[:b, :b] = Q[j].T
        big[b:, b:] = Q[j].T
        big[:b, b:] = dG[j]
        out[j] = _poly_cnp(big, k)[:b, b:]
    return out[0] if single else out


def backward(dy, x, W0, q_R, q_P, pi_R, pi_P, b: int, k: int):
    """Full backward to the compact parameters: (dx, dq_R, dq_P, dG_R, dG_P)."""
    Q_R = skew_from_params(q_R, b)
    Q_P = skew_from_params(q_P, b)
    G_R = neumann_cayley(Q_R, k)
    G_P = neumann_cayley(Q_P, k)
    dx, dG_R, dG_P = backward_from_blocks(dy, x, W0, G_R, G_P, pi_R, pi_P)
    dq_R = params_grad_from_skew_grad(cnp_vjp(Q_R, dG_R, k))
    dq_P = params_grad_from_skew_grad(cnp_vjp(Q_P, dG_P, k))
    return dx, dq_R, dq_P, dG_R, dG_P


# -------------------------------------------------------------- POET-XQ
def quantize_rows_int8(W):
    """Symmetric 8-bit storage of a weight, one scale per row (output channel):
    scale_i = max_j |W_ij| / 127 and q_ij = the integer nearest W_ij / scale_i
    (ties to even), in [-127, 127]; a row of zeros has scale 0 and codes 0.
    The codes are integers decided by floating point, so they are decided in
    float32, the precision the stored weight has (review Summary / Strengths,
    POET-XQ; the format itself is this library's reading).
    Returns (q int8 [m, n], scale float32 [m])."""
    W32 = np.asarray(W, dtype=np.float32)
    amax = np.max(np.abs(W32), axis=1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(W32 / safe[:, None])
    q = np.where(scale[:, None] > 0, q, 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, scale


def dequantize_rows(q, scale) -> np.ndarray:
    """The weight the quantized storage stands for: q_ij * scale_i (exact in float64)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[:, None]


# ------------------------------------------------------------------- merge
def merge(Wt, q_R, q_P, pi_R_old, pi_P_old, pi_R_new, pi_P_new, b: int, k: int):
    """Merge-then-reinitialize: fold R W0 P into the weight, resample the
    permutations and reset q (agidaily.cc article; review "merge_then_reinitialize").

    The stored weight is Wt = Pi_R W0 Pi_P^T, so W0 = Pi_R^T Wt Pi_P.  After the
    merge, W0' = R W0 P and the stored weight for the new permutations is
    Wt' = Pi_R' W0' Pi_P'^T.  Returns (Wt', q_R', q_P') with q' = 0."""
    Wt = np.asarray(Wt, dtype=np.float64)
    PR = gather_matrix(pi_R_old)
    PP = gather_matrix(pi_P_old)
    W0 = PR.T @ Wt @ PP
    G_R = blocks_from_params(q_R, b, k)
    G_P = blocks_from_params(q_P, b, k)
    W_eff = effective_weight(W0, G_R, G_P, pi_R_old, pi_P_old)
    Wt_new = gather_matrix(pi_R_new) @ W_eff @ gather_matrix(pi_P_new).T
    return Wt_new, np.zeros_like(np.asarray(q_R, dtype=np.float64)), \
        np.zeros_like(np.asarray(q_P, dtype=np.float64))


# ------------------------------------------ outputs the oracle computes one by one
# For full-size workloads the tests compare sampled outputs; each one is the
# same dense definition as above, restricted to the requested entries.
def input_grad(dy, W0, G_R, G_P, pi_R, pi_P) -> np.ndarray:
    """dX = dY R W0 P for the given rows of dY (rows are independent)."""
    R = orthogonal_from_blocks(G_R, pi_R)
    P = orthogonal_from_blocks(G_P, pi_P)
    return ((np.asarray(dy, dtype=np.float64) @ R) @ np.asarray(W0, dtype=np.float64)) @ P


def block_grad_entries(dy, x, W0, G_R, G_P, pi_R, pi_P, side: str, entries):
    """Selected entries (j, r, c) of dG_R or dG_P (see backward_from_blocks).

    dG_R,j[r, c] = dR[pi_R[jb+r], pi_R[jb+c]] with dR = dY^T X P^T W0^T, so
    dR[a, e] = dY[:, a] . (X P^T W0[e, :]^T);
    dG_P,j[r, c] = dP[pi_P[jb+r], pi_P[jb+c]] with dP = W0^T R^T dY^T X, so
    dP[a, e] = (dY R W0[:, a]) . X[:, e]."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    b = G_R.shape[-1]
    out = np.empty(len(entries))
    if side == "R":
        P = orthogonal_from_blocks(G_P, pi_P)
        pi = np.asarray(pi_R, dtype=np.int64)
        cache = {}
        for i, (j, r, c) in enumerate(entries):
            a, e = pi[j * b + r], pi[j * b + c]
            if e not in cache:
                cache[e] = x @ (P.T @ W0[e, :])
            out[i] = dy[:, a] @ cache[e]
    else:
        R = orthogonal_from_blocks(G_R, pi_R)
        pi = np.asarray(pi_P, dtype=np.int64)
        cache = {}
        for i, (j, r, c) in enumerate(entries):
            a, e = pi[j * b + r], pi[j * b + c]
            if a not in cache:
                cache[a] = dy @ (R @ W0[:, a])
            out[i] = cache[a] @ x[:, e]
    return out


def block_grad_blocks(dy, x, W0, G_R, G_P, pi_R, pi_P, side: str, blocks):
    """Whole blocks j of dG_R or dG_P (see backward_from_blocks).

    With idx = pi[jb : (j+1)b] the basis indices of block j,
    dG_R,j = dY[:, idx]^T (X P^T W0[idx, :]^T) and
    dG_P,j = (dY R W0[:, idx])^T X[:, idx]."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    b = G_R.shape[-1]
    out = np.empty((len(blocks), b, b))
    if side == "R":
        P = orthogonal_from_blocks(G_P, pi_P)
        pi = np.asarray(pi_R, dtype=np.int64)
        for t, j in enumerate(blocks):
            idx = pi[j * b:(j + 1) * b]
            out[t] = dy[:, idx].T @ (x @ (P.T @ W0[idx, :].T))
    else:
        R = orthogonal_from_blocks(G_R, pi_R)
        pi = np.asarray(pi_P, dtype=np.int64)
        for t, j in enumerate(blocks):
            idx = pi[j * b:(j + 1) * b]
            out[t] = (dy @ (R @ W0[:, idx])).T @ x[:, idx]
    return out


def merge_entries(Wt, G_R, G_P, pi_R_old, pi_P_old, pi_R_new, pi_P_new, entries):
    """Selected entries (i, j) of the merged stored weight
    Wt'[i, j] = (R W0 P)[pi_R_new[i], pi_P_new[j]] with W0 = Pi_R^T Wt Pi_P."""
    Wt = np.asarray(Wt, dtype=np.float64)
    R = orthogonal_from_blocks(G_R, pi_R_old)
    P = orthogonal_from_blocks(G_P, pi_P_old)
    inv_R = np.argsort(np.asarray(pi_R_old))   # W0[a, :] = Wt[inv_R[a], :] permuted
    inv_P = np.argsort(np.asarray(pi_P_old))
    W0 = Wt[inv_R][:, inv_P]
    out = np.empty(len(entries))
    for t, (i, j) in enumerate(entries):
        a, e = pi_R_new[i], pi_P_new[j]
        out[t] = R[a, :] @ W0 @ P[:, e]
    return out


# ------------------------------------------------------------ training step
# The step on either side of the layer: an optimizer update of the compact
# parameters, and merge-then-reinitialize on a fixed schedule.  The pages fix
# two numbers and no formula: the POET learning-rate scaling gamma = 0.5 and
# the POET reset gap of 400 steps (SAI replication review, Weaknesses, the
# single-run 8B/13B remark; the "Cayley approximation" remark ties gamma = 0.5
# to R - I ~ 2Q: a step in q moves R about twice as far).  The baseline
# optimizer throughout is AdamW.  Readings taken: q is updated by AdamW at the
# rate lr * gamma; weight decay is decoupled and 0 by default (decay on q would
# pull R towards I, not W towards 0); a merge (every reset gap updates) also
# zeroes the moments and restarts the bias-correction count, since q itself
# restarts from 0 in a new basis.
def adamw_step(q, g, m, v, t: int, lr: float, gamma: float = 0.5, beta1: float = 0.9, beta2: float = 0.999,
               eps: float = 1e-8, weight_decay: float = 0.0):
    """One AdamW update (Loshchilov and Hutter, "Decoupled Weight Decay
    Regularization", 2019, with the bias-corrected moment estimates of Kingma
    and Ba, "Adam", 2015) at the learning rate lr * gamma.  t >= 1 counts the
    updates since the moments were last reset.  Returns (q', m', v')."""
    q, g, m, v = (np.asarray(a, dtype=np.float64) for a in (q, g, m, v))
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    eta = lr * gamma
    q = q - eta * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * q)
    return q, m, v


def train_steps(xs, dys, W0, q_R, q_P, pi_R, pi_P, b: int, k: int, opt: dict, merge_every: int, new_perms):
    """Training steps of one layer for L_s = <dY_s, Y_s>: backward to dq,
    AdamW on (q_R, q_P), and after every `merge_every` updates a merge with the
    next permutation pair from `new_perms` (an iterator of (pi_R', pi_P'))
    followed by a reset of q, the moments and the count.  Returns
    (Wt, q_R, q_P, pi_R, pi_P) after the last step, Wt in the stored
    (pre-permuted) form."""
    Wt = prepermute(W0, pi_R, pi_P)
    q_R = np.asarray(q_R, dtype=np.float64)
    q_P = np.asarray(q_P, dtype=np.float64)
    mR, vR = np.zeros_like(q_R), np.zeros_like(q_R)
    mP, vP = np.zeros_like(q_P), np.zeros_like(q_P)
    t = 0
    for x, dy in zip(xs, dys):
        W0_cur = gather_matrix(pi_R).T @ Wt @ gather_matrix(pi_P)
        _, dq_R, dq_P, _, _ = backward(dy, x, W0_cur, q_R, q_P, pi_R, pi_P, b, k)
        t += 1
        q_R, mR, vR = adamw_step(q_R, dq_R, mR, vR, t, **opt)
        q_P, mP, vP = adamw_step(q_P, dq_P, mP, vP, t, **opt)
        if t == merge_every:
            pi_R_new, pi_P_new = next(new_perms)
            Wt, q_R, q_P = merge(Wt, q_R, q_P, pi_R, pi_P, pi_R_new, pi_P_new, b, k)
            pi_R, pi_P = pi_R_new, pi_P_new
            mR, vR, mP, vP = (np.zeros_like(a) for a in (mR, vR, mP, vP))
            t = 0
    return Wt, q_R, q_P, pi_R, pi_P
