"""Mem-SGD iterate on a strongly convex quadratic (oracle, test infrastructure).

Source: "Sparsified SGD with Memory", method section: x_{t+1} = x_t - g_t with
g_t = comp_k(m_t + eta_t grad_t), m_{t+1} = m_t + eta_t grad_t - g_t, step size
eta_t = 8 / (mu (a + t)), and the claim that with memory the method converges
at the rate of vanilla SGD (results section).

The shift ``a`` is not defined on the pages; it is an argument here.  Noise is
passed in (one row per step) so that the compressed and the uncompressed runs
see the same stochastic gradients.  Everything is float64 -- this is the
algorithm, not the float32 kernel.  Pinned exactly by two identities of the
update (k = d is vanilla SGD bit for bit; x_t - m_t moves by exactly -eta_t
times the stochastic gradient, to float64 rounding) and qualitatively by the
convergence claim.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .topk_ef import magnitude_order


@dataclass
class QuadraticProblem:
    lam: np.ndarray      # curvatures lambda_i in [mu, L]
    xstar: np.ndarray    # minimiser

    def f(self, x):
        return 0.5 * float(np.sum(self.lam * (x - self.xstar) ** 2))

    def grad(self, x):
        return self.lam * (x - self.xstar)


def _topk64(v: np.ndarray, k: int) -> np.ndarray:
    out = np.zeros_like(v)
    sel = magnitude_order(v)[:k]
    out[sel] = v[sel]
    return out


def _subset64(v: np.ndarray, idx: np.ndarray) -> np.ndarray:
    out = np.zeros_like(v)
    out[idx] = v[idx]
    return out


def run_memsgd(prob: QuadraticProblem, x0: np.ndarray, noise: np.ndarray, sigma: float,
               k: int | None, mu: float, a: float, subsets: np.ndarray | None = None,
               trace: list | None = None):
    """Run len(noise) steps.  k=None means no compression (vanilla SGD).
    With ``subsets`` (one row of k coordinates per step) the compressor is
    rand-k on those coordinates instead of top-k.  With ``trace`` (a list),
    every step appends (eta_t, stochastic gradient, x_{t+1}, m_{t+1}).

    Returns (x_T, x_bar_T) where x_bar_T is the uniform average of x_1..x_T.
    """
    x = np.array(x0, np.float64)
    mem = np.zeros_like(x)
    xsum = np.zeros_like(x)
    for t in range(noise.shape[0]):
        eta = 8.0 / (mu * (a + t))
        grad = prob.grad(x) + sigma * noise[t]
        acc = mem + eta * grad
        if k is None:
            g = acc
        elif subsets is not None:
            g = _subset64(acc, subsets[t])
        else:
            g = _topk64(acc, k)
        mem = acc - g
        x = x - g
        xsum += x
        if trace is not None:
            trace.append((eta, grad, x.copy(), mem.copy()))
    return x, xsum / noise.shape[0]
