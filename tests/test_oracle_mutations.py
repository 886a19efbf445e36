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


def _entries_transposed(dy, x, W0, G_R, G_P, pi_R, pi_P, side, entries):
    return O.__dict__["_orig_entries"](dy, x, W0, G_R, G_P, pi_R, pi_P, side, [(j, c, r) for j, r, c in entries])


def _blocks_transposed(dy, x, W0, G_R, G_P, pi_R, pi_P, side, blocks):
    return np.swapaxes(O.__dict__["_orig_blocks"](dy, x, W0, G_R, G_P, pi_R, pi_P, side, blocks), -1, -2)


def _input_grad_r_transposed(dy, W0, G_R, G_P, pi_R, pi_P):
    return O.__dict__["_orig_igrad"](dy, W0, np.swapaxes(G_R, -1, -2), G_P, pi_R, pi_P)


def _merge_entries_old_perms(Wt, G_R, G_P, pi_R_old, pi_P_old, pi_R_new, pi_P_new, entries):
    return O.__dict__["_orig_merge_e"](Wt, G_R, G_P, pi_R_old, pi_P_old, pi_R_old, pi_P_new, entries)


def _adamw_no_bias_correction(q, g, m, v, t, **opt):
    # bias correction forgotten: the count is frozen at a value where it vanishes
    return O.__dict__["_orig_adamw"](q, g, m, v, 10 ** 6, **opt)


def _adamw_unscaled_rate(q, g, m, v, t, **opt):
    return O.__dict__["_orig_adamw"](q, g, m, v, t, **dict(opt, gamma=1.0))


def _adamw_ascent(q, g, m, v, t, **opt):
    q1, m1, v1 = O.__dict__["_orig_adamw"](q, g, m, v, t, **opt)
    return 2 * np.asarray(q, float) - q1, m1, v1


def _train_without_reset(xs, dys, W0, q_R, q_P, pi_R, pi_P, b, k, opt, merge_every, new_perms):
    # the moments and the count run on through the merge
    Wt = O.prepermute(W0, pi_R, pi_P)
    mR = vR = np.zeros_like(q_R)
    mP = vP = np.zeros_like(q_P)
    t = seg = 0
    for x, dy in zip(xs, dys):
        W0_cur = O.gather_matrix(pi_R).T @ Wt @ O.gather_matrix(pi_P)
        _, dq_R, dq_P, _, _ = O.backward(dy, x, W0_cur, q_R, q_P, pi_R, pi_P, b, k)
        t += 1
        seg += 1
        q_R, mR, vR = O.adamw_step(q_R, dq_R, mR, vR, t, **opt)
        q_P, mP, vP = O.adamw_step(q_P, dq_P, mP, vP, t, **opt)
        if seg == merge_every:
            pi_R2, pi_P2 = next(new_perms)
            Wt, q_R, q_P = O.merge(Wt, q_R, q_P, pi_R, pi_P, pi_R2, pi_P2, b, k)
            pi_R, pi_P, seg = pi_R2, pi_P2, 0
    return Wt, q_R, q_P, pi_R, pi_P


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
    ("block_grad_entries", _entries_transposed, "_orig_entries",
     [P.test_sampled_block_grads_match_finite_differences]),
    ("block_grad_blocks", _blocks_transposed, "_orig_blocks",
     [P.test_sampled_block_grads_match_finite_differences]),
    ("input_grad", _input_grad_r_transposed, "_orig_igrad",
     [P.test_sampled_input_grad_rows_brute_force]),
    ("merge_entries", _merge_entries_old_perms, "_orig_merge_e",
     [P.test_merge_entries_match_merged_function]),
    ("adamw_step", _adamw_no_bias_correction, "_orig_adamw",
     [P.test_adamw_constant_gradient_closed_form, P.test_adamw_matches_library_optimizer]),
    ("adamw_step", _adamw_unscaled_rate, "_orig_adamw",
     [P.test_adamw_constant_gradient_closed_form, P.test_train_step_decreases_the_loss_to_first_order]),
    ("adamw_step", _adamw_ascent, "_orig_adamw",
     [P.test_adamw_matches_library_optimizer, P.test_train_step_decreases_the_loss_to_first_order]),
    ("train_steps", _train_without_reset, None,
     [P.test_train_after_merge_starts_afresh]),
]


@pytest.mark.parametrize("name,mutant,orig_key,pins", MUTATIONS, ids=[f"{m[0]}-{m[1].__name__}" for m in MUTATIONS])
def test_pin_catches_mutation(monkeypatch, name, mutant, orig_key, pins):
    if orig_key:
        monkeypatch.setitem(O.__dict__, orig_key, getattr(O, name))
    monkeypatch.setattr(O, name, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
