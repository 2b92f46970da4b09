"""Rand-k with memory (oracle, CPU): invariants, the contraction in expectation,
and the Mem-SGD comparison with top-k on the strongly convex quadratic.

"Sparsified SGD with Memory", method section: rand-k is a k-contraction,
E||x - rand_k(x)||^2 = (1 - k/d) ||x||^2; results section: with memory both
top-k and rand-k match vanilla SGD's rate, top-k usually ahead.
"""
import numpy as np
import pytest

import gen
import oracle


def test_invariants_and_special_cases():
    d, k = 10_000, 250
    g = gen.gaussian_vector(d, 5)
    mem = gen.gaussian_vector(d, 6, 0.5)
    idx = gen.randk_indices(0, 0, d, k)
    r = oracle.randk_ef_step(mem, g, 0.1, idx)
    assert np.array_equal((r["mem"] + r["g"]).view(np.uint32), r["acc"].view(np.uint32))   # m' + g = acc, bitwise
    assert np.count_nonzero(r["g"]) == k and np.all(r["mem"][idx].view(np.uint32) == 0)      # +0.0 entries
    assert np.array_equal(r["val"], r["acc"][idx])
    full = oracle.randk_ef_step(mem, g, 0.1, np.arange(d, dtype=np.int32))                  # k = d: g = acc
    assert np.array_equal(full["g"], full["acc"]) and not np.any(full["mem"])
    with pytest.raises(ValueError):
        oracle.randk_ef_step(mem, g, 0.1, np.array([3, 3], np.int32))


def test_subsets_are_uniform():
    d, k, steps = 1000, 50, 400
    counts = np.zeros(d)
    for t in range(steps):
        idx = gen.randk_indices(0, t, d, k)
        assert idx.size == k and np.all(np.diff(idx) > 0) and idx[0] >= 0 and idx[-1] < d
        counts[idx] += 1
    expect = steps * k / d
    chi2 = float(np.sum((counts - expect) ** 2 / expect))
    assert chi2 < d + 6 * np.sqrt(2 * d)          # chi-square with d-1 dof, 6 sigma


def test_contraction_in_expectation():
    d, k, draws = 2000, 200, 400
    x = gen.gaussian_vector(d, 8).astype(np.float64)
    ratios = []
    for t in range(draws):
        idx = gen.randk_indices(1, t, d, k)
        y = x.copy()
        y[idx] = 0.0
        ratios.append(np.sum(y * y) / np.sum(x * x))
    assert abs(np.mean(ratios) - (1 - k / d)) < 0.005


@pytest.mark.parametrize("k", [10])
def test_memsgd_randk_converges_topk_ahead(k):
    d, mu, L, sigma = 100, 1.0, 10.0, 0.1
    kappa = L / mu
    r = gen.rng(0, gen.KIND_MISC, 91, k)
    lam = np.exp(r.uniform(np.log(mu), np.log(L), d))
    lam[0], lam[1] = mu, L
    xstar = r.standard_normal(d)
    x0 = np.zeros(d)
    prob = oracle.QuadraticProblem(lam, xstar)
    T = int(50 * (d / k) * np.sqrt(kappa))
    noise = r.standard_normal((T, d))
    subsets = np.stack([gen.randk_indices(2, t, d, k) for t in range(T)])
    a = max(d / k, 16 * kappa)
    x_top, _ = oracle.run_memsgd(prob, x0, noise, sigma, k, mu, a)
    x_rand, _ = oracle.run_memsgd(prob, x0, noise, sigma, k, mu, a, subsets=subsets)
    x_sgd, _ = oracle.run_memsgd(prob, x0, noise, sigma, None, mu, a)
    f0 = prob.f(x0)
    assert prob.f(x_rand) <= 1e-2 * f0                  # rand-k with memory converges
    assert prob.f(x_rand) <= 10.0 * prob.f(x_sgd)
    assert prob.f(x_top) <= prob.f(x_rand)              # top-k ahead of rand-k at equal k
