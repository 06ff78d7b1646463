"""Pins of the oracle's key basis (the definition and the subspace
iteration the library follows) against things other than themselves: a
matrix built from known singular vectors, keys turned by the input
generator's own rotation (complex multiplication), the Eckart-Young
optimality of the SVD, the closed form of the iteration as the Q factor of
(X^T X)^(q+1) start^T, its convergence to the singular vectors on a graded
spectrum, and rank deficiency.
"""
import numpy as np
import pytest

import oracle as O
from decode_attention_05_amd import synth


def _orthonormal(rng, n, k):
    return np.linalg.qr(rng.standard_normal((n, k)))[0]


def _keys_from_x(X, G, H, d, pos, theta):
    """k_post [1, G, N, H, d] from pre-RoPE rows X [N, D], rotated by the
    input generator's rotation (complex multiplication, not the oracle's)."""
    N = X.shape[0]
    kp = synth._model_rotate(X.reshape(N, G, H, d).transpose(1, 2, 0, 3).astype(np.float64), pos, theta)
    return kp.transpose(0, 2, 1, 3)[None].astype(np.float64)


def _model_rotate64(x, pos, theta):
    d = x.shape[-1]
    half = d // 2
    freq = np.power(theta, -np.arange(half, dtype=np.float64) * 2.0 / d)
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * np.outer(pos.astype(np.float64), freq))
    return np.concatenate([z.real, z.imag], axis=-1)


def _keys64(X, G, H, d, pos, theta):
    N = X.shape[0]
    kp = _model_rotate64(X.reshape(N, G, H, d).transpose(1, 2, 0, 3), pos, theta)
    return kp.transpose(0, 2, 1, 3)[None]


def test_basis_recovers_known_singular_vectors_through_the_rotation():
    rng = np.random.default_rng(40)
    G, H, d, N, r = 2, 2, 8, 60, 6
    D = G * H * d
    U = _orthonormal(rng, N, D)
    V = _orthonormal(rng, D, D)
    s = np.linspace(20.0, 1.0, D) ** 1.5            # distinct, decreasing
    X = (U * s) @ V.T
    pos = rng.permutation(5000)[:N]
    k_post = _keys64(X, G, H, d, pos, 10000.0)
    assert np.allclose(O.pre_rope_keys(k_post, pos[None], [N], 10000.0)[0], X, atol=1e-12)
    basis, sv = O.key_basis(k_post, pos[None], [N], 10000.0, r)
    assert np.allclose(sv[0], s[:r], rtol=1e-12)
    for i in range(r):                               # each row is +- the i-th singular vector
        assert abs(abs(basis[0, i] @ V[:, i]) - 1.0) < 1e-12
    # the input generator's float32 rotation agrees to its own rounding
    k32 = _keys_from_x(X.astype(np.float32), G, H, d, pos, 10000.0)
    assert np.allclose(O.pre_rope_keys(k32, pos[None], [N], 10000.0)[0], X, atol=1e-4)


def test_basis_is_energy_optimal():
    # Eckart-Young: no orthonormal r-basis captures more of ||X||_F^2 than
    # the top-r right singular vectors, and they capture sum_{i<r} s_i^2
    rng = np.random.default_rng(41)
    G, H, d, N, r = 1, 2, 8, 40, 5
    k_post = rng.standard_normal((1, G, N, H, d)) * np.linspace(0.2, 3.0, d)
    X = O.pre_rope_keys(k_post, None, [N], 500.0)[0]
    basis, sv = O.key_basis(k_post, None, [N], 500.0, r)
    Bm = basis[0]
    assert np.allclose(Bm @ Bm.T, np.eye(r), atol=1e-12)
    e_opt = np.sum((X @ Bm.T) ** 2)
    assert e_opt == pytest.approx(np.sum(sv[0] ** 2), rel=1e-12)
    s_all = np.linalg.svd(X, compute_uv=False)
    assert e_opt == pytest.approx(np.sum(s_all[:r] ** 2), rel=1e-12)
    for _ in range(20):
        Rb = _orthonormal(rng, G * H * d, r).T
        assert np.sum((X @ Rb.T) ** 2) < e_opt
        Pb = np.linalg.qr((Bm + 0.01 * rng.standard_normal(Bm.shape)).T)[0].T
        assert np.sum((X @ Pb.T) ** 2) <= e_opt


def test_basis_padding_rows_and_rank_deficiency():
    rng = np.random.default_rng(42)
    G, H, d, N, r = 1, 2, 8, 12, 8
    k_post = rng.standard_normal((2, G, N, H, d))
    pos = np.stack([rng.permutation(100)[:N], rng.permutation(100)[:N]])
    basis, sv = O.key_basis(k_post, pos, [12, 5], 1e4, r)
    # sequence 1: rows >= 5 are padding -> only 5 singular vectors, the rest zero
    assert np.all(basis[1, 5:] == 0) and np.all(sv[1, 5:] == 0)
    b5, s5 = O.key_basis(k_post[1:, :, :5], pos[1:, :5], [5], 1e4, r)
    assert np.allclose(np.abs(basis[1, :5] @ b5[0, :5].T), np.eye(5), atol=1e-10)
    # the 5 rows span the row space: projecting reproduces X exactly
    X = O.pre_rope_keys(k_post, pos, [12, 5], 1e4)[1, :5]
    assert np.allclose(X @ basis[1].T @ basis[1], X, atol=1e-12)
    assert np.all(O.key_basis(k_post, pos, [0, 0], 1e4, r)[0] == 0)


def test_orth_columns_is_the_qr_factor_with_positive_diagonal():
    rng = np.random.default_rng(43)
    M = rng.standard_normal((9, 4))
    Q = O.orth_columns(M, 1e-5)
    assert np.allclose(Q.T @ Q, np.eye(4), atol=1e-13)
    R = Q.T @ M
    assert np.allclose(np.tril(R, -1), 0, atol=1e-13) and np.all(np.diag(R) > 0)
    assert np.allclose(Q @ R, M, atol=1e-13)
    # Gram-Schmidt by hand on two columns
    a, b = M[:, 0], M[:, 1]
    q0 = a / np.linalg.norm(a)
    w = b - (q0 @ b) * q0
    assert np.allclose(Q[:, 0], q0, atol=1e-14) and np.allclose(Q[:, 1], w / np.linalg.norm(w), atol=1e-13)
    # a dependent column is dropped; the later independent one still follows
    M2 = np.column_stack([a, 2.0 * a, b])
    Q2 = O.orth_columns(M2, 1e-5)
    assert np.all(Q2[:, 1] == 0)
    assert np.allclose(Q2[:, 0], q0, atol=1e-14) and np.allclose(np.abs(Q2[:, 2] @ Q[:, 1]), 1.0, atol=1e-12)
    # more columns than rows: the first n span R^n, the rest are dependent
    W = rng.standard_normal((3, 5))
    Q3 = O.orth_columns(W, 1e-5)
    assert np.allclose(Q3[:, :3].T @ Q3[:, :3], np.eye(3), atol=1e-13) and np.all(Q3[:, 3:] == 0)
    assert np.allclose(Q3[:, :3], O.orth_columns(W[:, :3], 1e-5), atol=1e-14)


@pytest.mark.parametrize("q", [0, 1, 2])
def test_iteration_closed_form(q):
    # Q = Q factor of (X^T X)^(q+1) start^T: intermediate orthonormalisations
    # multiply by upper-triangular factors only, which leave the Q factor alone
    rng = np.random.default_rng(44 + q)
    G, H, d, N, r = 1, 2, 8, 30, 4
    D = G * H * d
    U = _orthonormal(rng, N, D)
    V = _orthonormal(rng, D, D)
    X = (U * np.linspace(3.0, 1.0, D)) @ V.T          # well conditioned
    pos = np.arange(N) * 3
    k_post = _keys64(X, G, H, d, pos, 1e4)
    start = rng.standard_normal((1, r, D))
    got = O.key_basis_iteration(k_post, pos[None], [N], 1e4, start, q)[0]
    M = np.linalg.matrix_power(X.T @ X, q + 1) @ start[0].T
    Qm, Rm = np.linalg.qr(M)
    Qm = Qm * np.sign(np.diag(Rm))[None, :]
    assert np.allclose(got, Qm.T, atol=1e-10)


def test_iteration_converges_to_the_singular_vectors():
    rng = np.random.default_rng(47)
    G, H, d, N, r = 1, 2, 8, 50, 5
    D = G * H * d
    U = _orthonormal(rng, N, D)
    V = _orthonormal(rng, D, D)
    # graded spectrum: each singular value 1.6x the next
    X = (U * 1.6 ** -np.arange(D, dtype=np.float64)) @ V.T
    k_post = _keys64(X, G, H, d, np.arange(N), 1e4)
    start = rng.standard_normal((1, r, D))
    got = O.key_basis_iteration(k_post, None, [N], 1e4, start, 40)[0]
    ref, _ = O.key_basis(k_post, None, [N], 1e4, r)
    for i in range(r):
        assert abs(abs(got[i] @ ref[0, i]) - 1.0) < 1e-10
    # a spectrum with a gap at r: the subspace is found after few rounds
    s = np.concatenate([np.full(r, 10.0) + np.arange(r), np.full(D - r, 0.01)])
    X2 = (U * s) @ V.T
    k2 = _keys64(X2, G, H, d, np.arange(N), 1e4)
    got2 = O.key_basis_iteration(k2, None, [N], 1e4, start, 2)[0]
    P_ref = V[:, :r] @ V[:, :r].T
    assert np.max(np.abs(got2.T @ got2 - P_ref)) < 1e-10


def test_iteration_rank_deficiency_and_energy():
    rng = np.random.default_rng(48)
    G, H, d, N, r = 2, 2, 8, 20, 10
    D = G * H * d
    k_post = rng.standard_normal((2, G, N, H, d))
    start = rng.standard_normal((2, r, D))
    got = O.key_basis_iteration(k_post, None, [20, 6], 1e4, start, 2)
    X = O.pre_rope_keys(k_post, None, [20, 6], 1e4)
    # sequence 1 has rank 6: six orthonormal rows spanning its rows, four zero rows
    assert np.all(got[1, 6:] == 0)
    assert np.allclose(got[1, :6] @ got[1, :6].T, np.eye(6), atol=1e-12)
    assert np.allclose(X[1, :6] @ got[1].T @ got[1], X[1, :6], atol=1e-12)
    # sequence 0: orthonormal, and at most the optimum energy (Eckart-Young)
    assert np.allclose(got[0] @ got[0].T, np.eye(r), atol=1e-12)
    ref, sv = O.key_basis(k_post, None, [20, 6], 1e4, r)
    e = np.sum((X[0] @ got[0].T) ** 2)
    assert e <= np.sum(sv[0] ** 2) * (1 + 1e-12) and e > 0.9 * np.sum(sv[0] ** 2)
    # scale invariance, and the sequences do not interact
    got_s = O.key_basis_iteration(k_post * 1e3, None, [20, 6], 1e4, start, 2)
    assert np.allclose(got_s, got, atol=1e-10)
    one = O.key_basis_iteration(k_post[1:], None, [6], 1e4, start[1:], 2)
    assert np.array_equal(one[0], got[1])


def test_iteration_on_the_synthetic_recipe_captures_nearly_the_optimum():
    # low rank plus noise keys (the workload recipe): two power rounds leave
    # at most a few percent more residual energy than the SVD
    s = synth.scaled(synth.CONFIGS[1], batch=1, context=300, tail=16, rank=32, latent_rank=16)
    w = synth.make_workload(s, 49, with_basis=False)
    start = np.random.default_rng(50).standard_normal((1, s.rank, s.D))
    X = O.pre_rope_keys(w.k_post, w.pos, w.n_body, s.theta)[0]
    got = O.key_basis_iteration(w.k_post, w.pos, w.n_body, s.theta, start, 2)[0]
    ref, sv = O.key_basis(w.k_post, w.pos, w.n_body, s.theta, s.rank)
    total = np.sum(X ** 2)
    resid_opt = total - np.sum(sv[0] ** 2)
    resid = total - np.sum((X @ got.T) ** 2)
    assert resid_opt <= resid <= 1.10 * resid_opt
