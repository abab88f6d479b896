"""Pins for the oracle's per-block SVD (one-sided Jacobi).

The pages fix only that every K block and every V block gets its own SVD
(evolve.pub review, Summary).  The SVD itself is a textbook object, so the
oracle is pinned by what mathematics fixes: planted exact spectra, the LAPACK
routine, Weyl's perturbation bound, orthogonality and closed-form special cases.
"""
import numpy as np
import pytest
import torch

from synthetic import planted_blocks


def _planted_exact(n, T, d, seed):
    """Noise-free planted blocks plus their exact spectra (computed here from the
    same recipe: s_i = exp(-i / tau))."""
    X, tau = planted_blocks(n, T, d, (4.0, 32.0), seed, noise_std=0.0, out_dtype="f64",
                            return_tau=True)
    s = np.exp(-np.arange(d)[None, :] / tau.numpy()[:, None])
    return X.numpy(), s


@pytest.mark.parametrize("T", [128, 256, 512])
def test_planted_spectrum_recovered(oracle_lib, T):
    X, s = _planted_exact(3, T, 128, seed=11 + T)
    sigma, V, sweeps = oracle_lib.svd_blocks(X)
    assert (sweeps > 0).all()
    # s_0 = 1 for every planted block, so the bound is absolute.
    assert np.abs(sigma - s).max() <= 1e-12


def test_matches_lapack(oracle_lib):
    X = planted_blocks(4, 256, 128, (4.0, 32.0), 5, out_dtype="f64").numpy()
    sigma, V, _ = oracle_lib.svd_blocks(X)
    for b in range(X.shape[0]):
        ref = np.linalg.svd(X[b], compute_uv=False)
        assert np.abs(sigma[b] - ref).max() <= 1e-12 * ref[0]


def test_weyl_bound_under_noise(oracle_lib):
    n, T, d = 3, 256, 128
    X0, s = _planted_exact(n, T, d, seed=3)
    rng = np.random.default_rng(7)
    E = 1e-3 * rng.standard_normal((n, T, d))
    sigma, _, _ = oracle_lib.svd_blocks(X0 + E)
    for b in range(n):
        bound = np.linalg.norm(E[b], 2)
        assert np.abs(sigma[b] - s[b]).max() <= bound + 1e-12


def test_right_vectors_orthonormal_and_diagonalise(oracle_lib):
    X = planted_blocks(2, 256, 128, (4.0, 32.0), 9, out_dtype="f64").numpy()
    sigma, V, _ = oracle_lib.svd_blocks(X)
    for b in range(2):
        Vb = V[b]
        assert np.abs(Vb.T @ Vb - np.eye(128)).max() <= 1e-13
        # X^T X V = V diag(sigma^2): v_i are the right singular vectors.
        G = X[b].T @ X[b]
        resid = G @ Vb - Vb * sigma[b] ** 2
        assert np.abs(resid).max() <= 1e-12 * sigma[b][0] ** 2


def test_sign_convention(oracle_lib):
    X = planted_blocks(2, 256, 128, (4.0, 32.0), 10, out_dtype="f64").numpy()
    _, V, _ = oracle_lib.svd_blocks(X)
    for b in range(2):
        idx = np.argmax(np.abs(V[b]), axis=0)
        assert (V[b][idx, np.arange(128)] > 0).all()


def test_full_rank_reconstruction(oracle_lib):
    X = planted_blocks(1, 256, 128, (4.0, 32.0), 12, out_dtype="f64").numpy()[0]
    sigma, V, _ = oracle_lib.svd_blocks(X[None])
    A, B = oracle_lib.project(X, V[0], 128)
    assert np.abs(oracle_lib.reconstruct(A, B) - X).max() <= 1e-12
    # A = X V = U Sigma: its column norms are the singular values.
    assert np.abs(np.linalg.norm(A, axis=0) - sigma[0]).max() <= 1e-12


def test_special_cases(oracle_lib):
    d = 128
    # Zero block: every singular value 0, V = I.
    sigma, V, sweeps = oracle_lib.svd_blocks(np.zeros((1, 256, d)))
    assert (sigma == 0).all() and np.array_equal(V[0], np.eye(d)) and sweeps[0] == 1
    # Rank one: sigma_0 = |x| |y|, the rest 0.
    rng = np.random.default_rng(1)
    x, y = rng.standard_normal(256), rng.standard_normal(d)
    sigma, _, _ = oracle_lib.svd_blocks(np.outer(x, y)[None])
    assert abs(sigma[0, 0] - np.linalg.norm(x) * np.linalg.norm(y)) <= 1e-12 * sigma[0, 0]
    assert np.abs(sigma[0, 1:]).max() <= 1e-12 * sigma[0, 0]
    # Diagonal with distinct magnitudes: singular values are the sorted |diag|.
    D = np.zeros((256, d))
    diag = rng.permutation(np.linspace(-2.0, 3.0, d))
    D[np.arange(d), np.arange(d)] = diag
    sigma, _, _ = oracle_lib.svd_blocks(D[None])
    assert np.allclose(sigma[0], np.sort(np.abs(diag))[::-1], atol=1e-14)
    # Orthonormal columns: all singular values 1 (a fully degenerate spectrum).
    Q, _ = np.linalg.qr(rng.standard_normal((256, d)))
    sigma, _, _ = oracle_lib.svd_blocks(Q[None])
    assert np.abs(sigma - 1).max() <= 1e-13


def test_nonconvergence_is_reported(oracle_lib):
    X = planted_blocks(1, 256, 128, (4.0, 32.0), 13, out_dtype="f64").numpy()
    _, _, sweeps = oracle_lib.svd_blocks(X, max_sweeps=1)
    assert sweeps[0] == -1


def test_thread_count_does_not_change_results(oracle_lib):
    """Blocks are independent, so the OpenMP schedule cannot change any bit."""
    X = planted_blocks(6, 256, 128, (4.0, 32.0), 14, out_dtype="f64").numpy()
    s_all, V_all, _ = oracle_lib.svd_blocks(X)
    for b in range(6):
        s1, V1, _ = oracle_lib.svd_blocks(X[b:b + 1])
        assert np.array_equal(s1[0], s_all[b]) and np.array_equal(V1[0], V_all[b])


def test_bf16_input_is_widened_exactly(oracle_lib):
    """The oracle consumes the exact stored values: bf16 inputs widen without change."""
    Xb = planted_blocks(1, 256, 128, (4.0, 24.0), 15, out_dtype="bf16")
    X64 = Xb.to(torch.float64).numpy()
    s1, _, _ = oracle_lib.svd_blocks(Xb.float().numpy())
    s2, _, _ = oracle_lib.svd_blocks(X64)
    assert np.array_equal(s1, s2)
