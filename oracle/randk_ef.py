"""Mem-SGD rand-k compression with error-feedback memory (oracle, test infrastructure).

Source: "Sparsified SGD with Memory", method section -- the same update as
top-k, g_t = comp_k(m_t + eta_t grad_t), m_{t+1} = m_t + eta_t grad_t - g_t,
with comp_k = rand-k: keep k coordinates chosen uniformly at random (the page
names top-k and random-k as the two k-contraction operators; results section:
both match the rate of vanilla SGD, top-k usually ahead).

Readings taken:
  * rand-k keeps the chosen entries unscaled (a k-contraction, as the memory
    analysis needs) and zeroes the rest;
  * the random k-subset is an input (sorted, distinct indices): the method's
    random draws are made by the caller, so the oracle and the GPU see the
    same subset;
  * the accumulate, the message format and the +0.0 memory entries are those
    of the top-k oracle.
"""
from __future__ import annotations

import numpy as np

from .topk_ef import ef_accumulate


def randk_ef_step(mem: np.ndarray, grad: np.ndarray, eta: float, idx: np.ndarray) -> dict:
    """One rand-k step on the subset `idx` (strictly ascending, within [0, d))."""
    acc = ef_accumulate(mem, grad, eta)
    idx = np.asarray(idx, np.int64)
    if idx.size and (idx[0] < 0 or idx[-1] >= acc.size or np.any(np.diff(idx) <= 0)):
        raise ValueError("idx must be strictly ascending within [0, d)")
    val = acc[idx].copy()
    g = np.zeros_like(acc)
    g[idx] = val
    mem_new = acc.copy()
    mem_new[idx] = acc[idx] - acc[idx]          # +0.0
    return {"acc": acc, "idx": idx.astype(np.int32), "val": val, "g": g, "mem": mem_new}
