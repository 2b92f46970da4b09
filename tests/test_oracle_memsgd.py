"""Mem-SGD convergence on a strongly convex quadratic (CPU only).

"Sparsified SGD with Memory", method section: with memory and step size
eta_t = 8/(mu(a+t)), top-k SGD converges at the rate of vanilla SGD once
T = Omega(d/k * sqrt(kappa)); results section: the same rate for 0 < k <= d.
The shift a is undefined on the pages; a = max(d/k, 16 kappa) keeps
eta_0 * L <= 1/2.  The constants of the pass criterion are this test's own: a
qualitative pin (parity unpinned beyond it).
"""
import numpy as np
import pytest

import gen
import oracle


@pytest.mark.parametrize("k", [1, 10])
def test_memsgd_matches_sgd_rate(k):
    d, mu, L, sigma = 100, 1.0, 10.0, 0.1
    kappa = L / mu
    r = gen.rng(0, gen.KIND_MISC, 90, k)
    lam = np.exp(r.uniform(np.log(mu), np.log(L), d))
    lam[0], lam[1] = mu, L
    xstar = r.standard_normal(d)
    x0 = np.zeros(d)
    prob = oracle.QuadraticProblem(lam, xstar)
    T = int(50 * (d / k) * np.sqrt(kappa))
    noise = r.standard_normal((T, d))
    a = max(d / k, 16 * kappa)
    x_mem, xbar_mem = oracle.run_memsgd(prob, x0, noise, sigma, k, mu, a)
    x_sgd, _ = oracle.run_memsgd(prob, x0, noise, sigma, None, mu, a)
    f0 = prob.f(x0)
    gap_mem, gap_sgd = prob.f(x_mem), prob.f(x_sgd)
    assert gap_mem <= 3.0 * gap_sgd
    assert gap_mem <= 1e-2 * f0
    assert prob.f(xbar_mem) < f0       # informational average (weights unspecified): only sanity


def test_memory_is_what_makes_it_converge():
    """Dropping the memory (plain top-k SGD) is far worse at small k: the pin is sensitive to it."""
    d, mu, L, sigma, k = 100, 1.0, 10.0, 0.1, 1
    r = gen.rng(0, gen.KIND_MISC, 91)
    lam = np.exp(r.uniform(np.log(mu), np.log(L), d))
    xstar = r.standard_normal(d)
    prob = oracle.QuadraticProblem(lam, xstar)
    T = 3000
    noise = r.standard_normal((T, d))
    a = max(d / k, 16 * L / mu)
    x_mem, _ = oracle.run_memsgd(prob, np.zeros(d), noise, sigma, k, mu, a)
    # no memory: x -= top_k(eta * grad)
    x = np.zeros(d)
    for t in range(T):
        eta = 8.0 / (mu * (a + t))
        v = eta * (prob.grad(x) + sigma * noise[t])
        sel = oracle.magnitude_order(v)[:k]
        x[sel] -= v[sel]
    assert prob.f(x_mem) < 0.5 * prob.f(x)
