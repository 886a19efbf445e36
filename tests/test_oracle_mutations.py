"""The pins must catch plausible mistakes: each case plants one mistake in the
oracle (on the CPU, through monkeypatch) and checks that a pin then fails."""
import numpy as np
import pytest

from oracle import poet_oracle as O
from tests import test_oracle_pins as P


def _pack_sign_flip(dQ):
    return -O.__dict__["_orig_pack"](dQ)


def _triangle_column_major(b):
    return [(r, c) for c in range(b) for r in range(c)]


def _neumann_off_by_one(Q, k):
    return O.__dict__["_orig_neumann"](Q, k - 1)


def _forward_transposed(x, W0, G_R, G_P, pi_R, pi_P):
    R = O.orthogonal_from_blocks(G_R, pi_R)
    P = O.orthogonal_from_blocks(G_P, pi_P)
    return np.asarray(x, float) @ P @ np.asarray(W0, float).T @ R.T


def _orth_inverse_perm(G, pi):
    D = O.block_diag(G)
    pi = np.asarray(pi)
    return D[np.ix_(pi, pi)]


def _vjp_without_transpose(Q, dG, k):
    Qt = np.swapaxes(np.asarray(Q, float), -1, -2)
    return O.__dict__["_orig_vjp"](Qt, dG, k)


def _backward_block_transposed(dy, x, W0, G_R, G_P, pi_R, pi_P):
    dx, dG_R, dG_P = O.__dict__["_orig_bwd"](dy, x, W0, G_R, G_P, pi_R, pi_P)
    return dx, np.swapaxes(dG_R, -1, -2), dG_P


MUTATIONS = [
    ("params_grad_from_skew_grad", _pack_sign_flip, "_orig_pack",
     [P.test_skew_exact_and_pack_adjoint]),
    ("triangle_pairs", _triangle_column_major, None,
     [lambda: P.test_skew_layout_golden("skew_b4.txt", 4)]),
    ("neumann_cayley", _neumann_off_by_one, "_orig_neumann",
     [P.test_cnp_b2_golden, lambda: P.test_cnp_singular_values(3)]),
    ("forward_from_blocks", _forward_transposed, None,
     [P.test_input_centric_chain_matches_dense]),
    ("orthogonal_from_blocks", _orth_inverse_perm, None,
     [P.test_orthogonal_from_blocks_is_conjugation, P.test_input_centric_chain_matches_dense]),
    ("cnp_vjp", _vjp_without_transpose, "_orig_vjp",
     [P.test_cnp_vjp_matches_finite_differences, lambda: P.test_backward_matches_finite_differences(3)]),
    ("backward_from_blocks", _backward_block_transposed, "_orig_bwd",
     [lambda: P.test_backward_matches_finite_differences(3)]),
]


@pytest.mark.parametrize("name,mutant,orig_key,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_mutation(monkeypatch, name, mutant, orig_key, pins):
    if orig_key:
        monkeypatch.setitem(O.__dict__, orig_key, getattr(O, name))
    monkeypatch.setattr(O, name, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
