"""Pins of the equal-budget comparison allocations (uniform, random) that the
greedy is ablated against (evolve.pub review of arXiv 2609.29913, Strengths:
Fig. 5(d) compares entropy-based allocation with uniform and random allocation
at the same budget).

  * SplitMix64, the counter-based generator of the random keys, against a
    published output of its reference definition and the uniformity of its
    high 32 bits;
  * uniform = the literal greedy on a pool of identical spectra (whose ties go
    to the smaller block), and its closed-form properties;
  * random = a uniformly random subset of the pool's (block, index) slots: the
    budget is spent exactly, ranks respect the caps, and over many seeds every
    block's rank has the mean and variance of the hypergeometric law;
  * the greedy's objective is the largest of the three at every budget
    (the greedy is optimal for the separable concave objective).
"""
import numpy as np
import pytest

import oracle


def test_splitmix64_reference_output():
    # First output of SplitMix64 seeded with 0 (Java's SplittableRandom(0).nextLong()
    # is -2152535657050944081, the same 64 bits as a signed integer).
    assert oracle.splitmix64(0, 1) == 0xE220A8397B1DCDAF
    assert oracle.splitmix64(0, 1) - 2**64 == -2152535657050944081


def test_splitmix64_high_bits_are_uniform():
    keys = np.array([oracle.splitmix64(12345, c) >> 32 for c in range(1, 40001)], dtype=np.uint64)
    hist = np.bincount((keys >> np.uint64(26)).astype(np.int64), minlength=64)  # 64 bins
    expect = len(keys) / 64
    chi2 = float(((hist - expect) ** 2 / expect).sum())
    assert chi2 < 120.0, chi2  # 63 degrees of freedom: p(chi2 > 120) < 1e-5
    assert len(np.unique(keys)) > len(keys) - 5


@pytest.mark.parametrize("n,k,R", [(5, 8, 0), (5, 8, 3), (5, 8, 17), (5, 8, 40), (5, 8, 99), (1, 128, 64),
                                   (32, 128, 2048), (7, 128, 100)])
def test_uniform_is_the_greedy_on_identical_spectra(n, k, R):
    sigma = np.tile(np.linspace(1.0, 0.1, k), (n, 1))
    greedy, _, _ = oracle.allocate(sigma, R, 1e-4)
    uni, _ = oracle.allocate_policy(sigma, R, 1e-4, "uniform")
    np.testing.assert_array_equal(uni, greedy)
    assert uni.sum() == min(R, n * k)
    assert uni.max() - uni.min() <= 1 and np.all(np.diff(uni) <= 0)


@pytest.mark.parametrize("n,k,R", [(4, 8, 0), (4, 8, 5), (4, 8, 31), (4, 8, 32), (4, 8, 50), (64, 128, 4096)])
def test_random_spends_the_budget_within_caps(n, k, R):
    sigma = np.ones((n, k))
    for seed in range(5):
        r, _ = oracle.allocate_policy(sigma, R, 1e-4, "random", seed=seed)
        assert r.sum() == min(R, n * k)
        assert r.min() >= 0 and r.max() <= k


def test_random_depends_on_seed_and_pool():
    sigma = np.ones((16, 128))
    a, _ = oracle.allocate_policy(sigma, 1024, 1e-4, "random", seed=1, pool=0)
    b, _ = oracle.allocate_policy(sigma, 1024, 1e-4, "random", seed=2, pool=0)
    c, _ = oracle.allocate_policy(sigma, 1024, 1e-4, "random", seed=1, pool=1)
    d, _ = oracle.allocate_policy(sigma, 1024, 1e-4, "random", seed=1, pool=0)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    np.testing.assert_array_equal(a, d)


def test_random_matches_the_hypergeometric_law():
    # R of N = n k slots drawn without replacement: a block's rank is
    # hypergeometric(N, k, R) with mean k R / N and variance
    # R (k/N) (1 - k/N) (N - R) / (N - 1).
    n, k, R = 8, 16, 40
    N = n * k
    ranks = np.array([oracle.allocate_policy(np.ones((n, k)), R, 1e-4, "random", seed=s)[0]
                      for s in range(3000)], dtype=np.float64)
    mean = k * R / N
    var = R * (k / N) * (1 - k / N) * (N - R) / (N - 1)
    assert np.all(np.abs(ranks.mean(axis=0) - mean) < 5 * np.sqrt(var / len(ranks)))
    assert np.all(np.abs(ranks.var(axis=0) / var - 1) < 0.12)


@pytest.mark.parametrize("frac", [0.25, 0.5, 0.75])
def test_greedy_objective_is_the_largest(frac):
    rng = np.random.default_rng(7)
    n, k = 24, 128
    tau = rng.uniform(4, 64, size=n)
    sigma = np.exp(-np.arange(k)[None, :] / tau[:, None]) + 1e-3 * rng.random((n, k))
    sigma = -np.sort(-sigma, axis=1)
    R = int(frac * n * k)
    objs = {pol: oracle.allocate_policy(sigma, R, 1e-4, pol, seed=3)[1] for pol in oracle.POLICIES}
    assert objs["entropy"] >= objs["uniform"] and objs["entropy"] >= objs["random"]
    assert objs["entropy"] > objs["uniform"] * (1 + 1e-6)
