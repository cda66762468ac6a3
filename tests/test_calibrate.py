"""Host-side basis calibration (sparse_attention_long_kv_amd.calibrate).

The pages do not name the calibration matrix, so these tests pin what the
mathematics fixes: orthonormal bases, the closed-form optimum when query and
key moments share eigenvectors, exact scores for rank-r keys and isotropic
queries, rotation equivariance, and that the chosen basis never has a larger
score error than the other candidates or a random basis.
"""

import numpy as np

from sparse_attention_long_kv_amd.calibrate import (basis_candidates, basis_from_moments,
                                                    calibrate_basis, score_error,
                                                    score_moments)


def _rot(d, seed):
    q, r = np.linalg.qr(np.random.default_rng(seed).standard_normal((d, d)))
    return q * np.sign(np.diag(r))[None, :]


def _proj(P):
    return P @ P.T


def test_bases_are_orthonormal():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((300, 32)) * np.linspace(2, 0.1, 32)
    k = rng.standard_normal((900, 32)) * np.linspace(0.1, 2, 32)
    for P in basis_candidates(*score_moments(q, k), 8).values():
        assert np.allclose(P.T @ P, np.eye(8), atol=1e-12)
    P, _ = calibrate_basis(q, k, 8)
    assert P.shape == (32, 8) and np.allclose(P.T @ P, np.eye(8), atol=1e-12)


def test_shared_eigenvectors_give_the_closed_form_optimum():
    """C_q = U diag(a) U^T, C_k = U diag(b) U^T: E(Pi) = sum of the dropped
    a_i b_i over sum a_i b_i, minimal for the r largest products."""
    d, r = 24, 6
    U = _rot(d, 2)
    i = np.arange(d)
    a = 1.0 / (1.0 + np.abs(i - 12.0))          # queries weigh the middle directions
    b = np.exp(-i / 6.0)                        # keys carry most energy early
    c_q, c_k = U @ np.diag(a) @ U.T, U @ np.diag(b) @ U.T
    top = np.argsort(a * b)[::-1][:r]
    P_opt = U[:, top]
    e_opt = (np.sum(a * b) - np.sum((a * b)[top])) / np.sum(a * b)
    assert abs(score_error(P_opt, c_q, c_k) - e_opt) < 1e-12
    P, rep = basis_from_moments(c_q, c_k, r)
    assert np.allclose(_proj(P), _proj(P_opt), atol=1e-9)
    assert abs(rep["relative_score_error"][rep["chosen"]] - e_opt) < 1e-12
    # key moments alone keep the r most energetic key directions: worse here
    assert rep["relative_score_error"]["key_moments"] > e_opt + 1e-3


def test_rank_r_keys_and_isotropic_queries_score_exactly():
    d, r = 32, 5
    rng = np.random.default_rng(3)
    A = _rot(d, 4)[:, :r]
    keys = rng.standard_normal((2000, r)) @ A.T + 0.7    # a mean shift is allowed
    q = rng.standard_normal((4000, d))
    P, rep = calibrate_basis(q, keys, r)
    assert rep["relative_score_error"][rep["chosen"]] < 1e-20
    qt = rng.standard_normal((7, d))
    kc = keys[:50] - keys.mean(axis=0)
    assert np.allclose((qt @ P) @ (P.T @ kc.T), qt @ kc.T, atol=1e-9)


def test_rotation_equivariance():
    d, r = 20, 4
    rng = np.random.default_rng(5)
    q = rng.standard_normal((500, d)) * np.linspace(1.5, 0.2, d)
    k = rng.standard_normal((800, d)) * np.linspace(0.3, 1.2, d)
    R = _rot(d, 6)
    P, rep = calibrate_basis(q, k, r)
    P2, rep2 = calibrate_basis(q @ R.T, k @ R.T, r)
    assert rep["chosen"] == rep2["chosen"]
    assert np.allclose(_proj(P2), R @ _proj(P) @ R.T, atol=1e-8)


def test_chosen_basis_has_the_smallest_error():
    d, r = 48, 8
    rng = np.random.default_rng(7)
    U = _rot(d, 8)
    i = np.arange(d)
    q = (rng.standard_normal((600, d)) * np.sqrt(1.0 / (1.0 + np.abs(i - 20) / 3.0))) @ U.T
    k = (rng.standard_normal((3000, d)) * np.sqrt(1.0 / (1.0 + i / 3.0))) @ U.T
    c_q, c_k = score_moments(q, k)
    P, rep = basis_from_moments(c_q, c_k, r)
    e = rep["relative_score_error"]
    assert e[rep["chosen"]] == min(e.values())
    rand = np.linalg.qr(rng.standard_normal((d, r)))[0]
    assert score_error(P, c_q, c_k) < score_error(rand, c_q, c_k)
