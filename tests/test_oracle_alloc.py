"""Pins for the oracle's rank allocation.

The pages define the allocation as maximising the spectral information
sum_b sum_{i < r_b} log(1 + sigma_{b,i}^2 / eps^2) under a global rank budget,
solved greedily by marginal gains (evolve.pub review, Strengths, Eqs 5-7).
Pins: exhaustive enumeration on tiny pools, the closed form of the greedy
(the R largest singular values in the order sigma desc, block asc, index asc),
and the special cases that closed form predicts.
"""
import itertools

import numpy as np
import pytest


def _random_pool(rng, n, k, distinct=True):
    s = rng.uniform(0.0, 2.0, size=(n, k))
    if not distinct:
        s = np.round(s * 4) / 4  # force ties
    return -np.sort(-s, axis=1)


def _brute_force(sigma, R, eps2):
    n, k = sigma.shape
    gains = np.log1p(sigma ** 2 / eps2)
    cum = np.concatenate([np.zeros((n, 1)), np.cumsum(gains, axis=1)], axis=1)
    best = -1.0
    best_alloc = []
    for alloc in itertools.product(range(k + 1), repeat=n):
        if sum(alloc) != min(R, n * k):
            continue
        val = sum(cum[b, alloc[b]] for b in range(n))
        if val > best + 1e-12:
            best, best_alloc = val, [alloc]
        elif abs(val - best) <= 1e-12:
            best_alloc.append(alloc)
    return best, best_alloc


@pytest.mark.parametrize("n,k", [(1, 6), (2, 5), (3, 4), (4, 3), (4, 6)])
def test_greedy_is_optimal_by_enumeration(oracle_lib, n, k):
    rng = np.random.default_rng(100 + 10 * n + k)
    eps2 = 0.05
    for trial in range(3):
        sigma = _random_pool(rng, n, k, distinct=(trial != 2))
        for R in range(0, n * k + 2):
            rank, obj, given = oracle_lib.allocate(sigma, R, eps2)
            best, allocs = _brute_force(sigma, R, eps2)
            assert given == min(R, n * k)
            assert int(rank.sum()) == min(R, n * k)
            assert abs(obj - best) <= 1e-10
            assert abs(oracle_lib.objective(sigma, rank, eps2) - obj) <= 1e-12
            if len(allocs) == 1:
                assert tuple(int(r) for r in rank) == allocs[0]
            else:
                assert tuple(int(r) for r in rank) in allocs


def _top_r(sigma, R):
    """The greedy's closed form: counts per block of the R largest keys (sigma desc, b asc, i asc)."""
    n, k = sigma.shape
    keys = sorted(((-sigma[b, i], b, i) for b in range(n) for i in range(k)))
    rank = np.zeros(n, dtype=np.int32)
    for _, b, _ in keys[:R]:
        rank[b] += 1
    return rank


def test_greedy_equals_top_r_of_sigma(oracle_lib):
    rng = np.random.default_rng(5)
    for _ in range(20):
        n = int(rng.integers(1, 12))
        k = int(rng.integers(1, 40))
        sigma = _random_pool(rng, n, k, distinct=bool(rng.integers(0, 2)))
        R = int(rng.integers(0, n * k + 3))
        rank, _, _ = oracle_lib.allocate(sigma, R, 1e-4)
        assert np.array_equal(rank, _top_r(sigma, R))


def test_equal_spectra_round_robin(oracle_lib):
    s = np.linspace(1.0, 0.1, 10)
    sigma = np.tile(s, (5, 1))
    for R in range(0, 51):
        rank, _, _ = oracle_lib.allocate(sigma, R, 1e-4)
        m, j = divmod(R, 5)
        expect = [m + 1] * j + [m] * (5 - j)
        assert list(rank) == expect


def test_budget_edges(oracle_lib):
    rng = np.random.default_rng(9)
    sigma = _random_pool(rng, 6, 16)
    rank, obj, given = oracle_lib.allocate(sigma, 0, 1e-4)
    assert (rank == 0).all() and obj == 0.0 and given == 0
    rank, obj, given = oracle_lib.allocate(sigma, 6 * 16 + 50, 1e-4)
    assert (rank == 16).all() and given == 96
    # Zero-gain increments are still handed out (budget spent exactly).
    # With every gain equal to zero the tie rule (smallest block first) fills
    # block 0, then block 1.
    z = np.zeros((3, 4))
    rank, obj, given = oracle_lib.allocate(z, 7, 1e-4)
    assert list(rank) == [4, 3, 0] and obj == 0.0 and given == 7


def test_eps_changes_objective_not_ranks(oracle_lib):
    rng = np.random.default_rng(21)
    sigma = _random_pool(rng, 8, 32)
    r1, o1, _ = oracle_lib.allocate(sigma, 100, 1e-4)
    r2, o2, _ = oracle_lib.allocate(sigma, 100, 1.0)
    r3, o3, _ = oracle_lib.allocate(sigma, 100, 1e-8)
    assert np.array_equal(r1, r2) and np.array_equal(r1, r3)
    assert o1 != o2 and o1 != o3


def test_planted_pool_ranks_follow_tau(oracle_lib):
    """Blocks with a slower-decaying planted spectrum (larger tau) get more rank."""
    from synthetic import planted_blocks
    X, tau = planted_blocks(8, 256, 128, (4.0, 32.0), 77, out_dtype="f64", return_tau=True)
    sigma, _, _ = oracle_lib.svd_blocks(X.numpy())
    rank, _, _ = oracle_lib.allocate(sigma, 512, 1e-4)
    assert int(rank.sum()) == 512
    t = tau.numpy()
    for a in range(8):
        for b in range(8):
            if t[a] > t[b] + 2.0:
                assert rank[a] >= rank[b]


def test_compress_several_pools(oracle_lib):
    """oracle.compress over a pool table with pools of unequal sizes and budgets
    (one pool empty, one budget zero): each pool's ranks are the greedy's closed
    form on that pool's own singular values and budget, the objective per pool
    is the sum of its selected gains, and every block's factors carry its own
    rank (the Eckart-Young residual of that rank)."""
    from synthetic import planted_blocks
    X = planted_blocks(9, 128, 128, (4.0, 32.0), 91, out_dtype="f64").numpy()
    pool_ptr, budgets, eps2 = [0, 2, 2, 6, 9], [100, 5, 300, 0], 1e-4
    comp = oracle_lib.compress(X, pool_ptr, budgets, eps2, "f32")
    assert len(comp.objective) == 4
    for p in range(4):
        lo, hi = pool_ptr[p], pool_ptr[p + 1]
        want = _top_r(comp.sigma[lo:hi], budgets[p]) if hi > lo else np.zeros(0, dtype=np.int32)
        assert np.array_equal(comp.rank[lo:hi], want), p
        gains = sum(np.log1p(comp.sigma[b, :comp.rank[b]] ** 2 / eps2).sum() for b in range(lo, hi))
        assert abs(comp.objective[p] - gains) <= 1e-9 * max(1.0, gains), p
    assert comp.rank[6:].sum() == 0 and comp.rank[2:6].sum() == 300 and comp.rank[:2].sum() == 100
    for b in range(9):
        r = int(comp.rank[b])
        assert comp.A[b].shape == (128, r) and comp.B[b].shape == (r, 128)
        err2 = np.sum((X[b] - comp.A[b] @ comp.B[b]) ** 2)
        assert abs(err2 - np.sum(comp.sigma[b, r:] ** 2)) <= 1e-6 * np.sum(comp.sigma[b] ** 2), b
