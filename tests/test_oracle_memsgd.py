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


def _problem(seed, d=60, mu=1.0, L=10.0):
    r = gen.rng(0, gen.KIND_MISC, seed)
    lam = np.exp(r.uniform(np.log(mu), np.log(L), d))
    return oracle.QuadraticProblem(lam, r.standard_normal(d)), r


def test_k_equal_d_is_vanilla_sgd():
    """With k = d the compressor keeps everything: g_t = m_t + eta_t grad_t,
    the memory stays zero and the iterate is SGD's, bit for bit."""
    prob, r = _problem(92)
    d = prob.lam.size
    noise = r.standard_normal((400, d))
    tr = []
    x_k, xb_k = oracle.run_memsgd(prob, np.zeros(d), noise, 0.1, d, 1.0, 16 * 10.0, trace=tr)
    x_s, xb_s = oracle.run_memsgd(prob, np.zeros(d), noise, 0.1, None, 1.0, 16 * 10.0)
    assert np.array_equal(x_k, x_s) and np.array_equal(xb_k, xb_s)
    assert all(not m.any() for _, _, _, m in tr)


@pytest.mark.parametrize("k,subsets", [(1, False), (7, False), (7, True)])
def test_virtual_iterate_moves_like_sgd(k, subsets):
    """Method section of "Sparsified SGD with Memory": the memory holds what
    was not yet applied, so x_{t+1} - m_{t+1} = x_t - m_t - eta_t grad_t exactly
    (here to float64 rounding) for any comp_k, top-k or rand-k; and the memory
    holds at most d - k nonzero entries after each top-k step."""
    prob, r = _problem(93)
    d, T = prob.lam.size, 600
    noise = r.standard_normal((T, d))
    sub = np.stack([np.sort(r.choice(d, k, replace=False)) for _ in range(T)]) if subsets else None
    tr = []
    x0 = r.standard_normal(d)
    oracle.run_memsgd(prob, x0, noise, 0.1, k, 1.0, max(d / k, 160.0), subsets=sub, trace=tr)
    v_prev = x0.copy()                       # x_0 - m_0, m_0 = 0
    for t, (eta, grad, x, m) in enumerate(tr):
        v = x - m
        want = v_prev - eta * grad
        scale = max(1.0, float(np.max(np.abs(v_prev))))
        assert np.max(np.abs(v - want)) <= 1e-13 * scale, f"step {t}"
        if not subsets:
            assert np.count_nonzero(m) <= d - k
        v_prev = v
    # a planted mistake (the memory keeps acc instead of acc - g) breaks the identity
    eta, grad, x, m = tr[10]
    _, _, x_prev, m_prev = tr[9]
    acc = m_prev + eta * grad
    assert np.max(np.abs((x - acc) - (x_prev - m_prev - eta * grad))) > 1e-6
