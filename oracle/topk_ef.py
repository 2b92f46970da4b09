"""Mem-SGD top-k compression with error-feedback memory (oracle, test infrastructure).

Source: "Sparsified SGD with Memory", method section -- the update
    g_t     = comp_k(m_t + eta_t * grad_t)
    m_{t+1} = m_t + eta_t * grad_t - g_t
and the abstract, where comp_k keeps the "most significant entries" (largest
magnitude) of the vector.  The pages fix neither the float format nor a tie
rule; the readings taken here are:

  * the accumulate is two float32 operations, each rounded once to nearest-even:
    t_i = fl32(eta * grad_i), acc_i = fl32(m_i + t_i).  The oracle forms each
    exact result in float64 and rounds it to float32 once; for a product of two
    float32 numbers float64 is exact, and for a sum the float64 intermediate
    has >= 2*24+2 bits so the double rounding equals a single float32 rounding;
  * selection order is (|acc| descending, index ascending): among equal
    magnitudes (including +x and -x) the lower index wins;
  * the message is (index int32, value float32) pairs in ascending index order;
  * a selected memory entry becomes acc_i - acc_i = +0.0.
"""
from __future__ import annotations

import numpy as np


def grad_to_f64(grad: np.ndarray) -> np.ndarray:
    """Gradient as float64.  uint16 arrays are bf16 bit patterns (widened exactly)."""
    g = np.asarray(grad)
    if g.dtype == np.uint16:
        return (g.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if g.dtype == np.float32:
        return g.astype(np.float64)
    raise TypeError(f"gradient dtype {g.dtype} not supported (float32 or bf16 bits as uint16)")


def ef_accumulate(mem: np.ndarray, grad: np.ndarray, eta: float) -> np.ndarray:
    """acc = m + eta*grad with each of the two operations rounded to float32."""
    eta64 = np.float64(np.float32(eta))
    step = (eta64 * grad_to_f64(grad).ravel()).astype(np.float32)          # fl32(eta*g)
    acc = (np.asarray(mem, np.float32).ravel().astype(np.float64)
           + step.astype(np.float64)).astype(np.float32)                     # fl32(m + .)
    return acc


def magnitude_order(acc: np.ndarray) -> np.ndarray:
    """All indices sorted by |acc| descending, equal magnitudes by index ascending.

    A stable sort on -|acc| keeps the original (ascending) index order among
    equal keys, which is exactly the tie rule.
    """
    mag = np.abs(np.asarray(acc).astype(np.float64))
    return np.argsort(-mag, kind="stable")


def topk_select(acc: np.ndarray, k: int) -> np.ndarray:
    """Indices of comp_k(acc) = top-k by magnitude, returned in ascending order."""
    d = acc.size
    if not (1 <= k <= d):
        raise ValueError("need 1 <= k <= d")
    return np.sort(magnitude_order(acc)[:k]).astype(np.int32)


def topk_ef_step(mem: np.ndarray, grad: np.ndarray, eta: float, k: int) -> dict:
    """One encode step of Mem-SGD with top-k.

    Returns acc, the message (idx ascending, val), the dense g_t and m_{t+1}.
    """
    acc = ef_accumulate(mem, grad, eta)
    idx = topk_select(acc, k)
    g_dense = np.zeros(acc.size, np.float32)
    g_dense[idx] = acc[idx]
    # m_{t+1} = (m_t + eta*grad) - g_t, the subtraction in float32 (exact here)
    mem_new = (acc.astype(np.float64) - g_dense.astype(np.float64)).astype(np.float32)
    return {"acc": acc, "idx": idx, "val": acc[idx].copy(), "g": g_dense, "mem": mem_new}


def topk_decode(idx: np.ndarray, val: np.ndarray, d: int, out: np.ndarray | None = None,
                accumulate: bool = False) -> np.ndarray:
    """Dense decode of the (index, value) message.

    accumulate=False: out = 0 everywhere, then out[idx] = val.
    accumulate=True : out[idx] = fl32(out[idx] + val) on a caller-provided out.
    """
    idx = np.asarray(idx, np.int64)
    val = np.asarray(val, np.float32)
    if accumulate:
        if out is None:
            raise ValueError("accumulate needs out")
        res = np.asarray(out, np.float32).copy()
        res[idx] = (res[idx].astype(np.float64) + val.astype(np.float64)).astype(np.float32)
        return res
    res = np.zeros(d, np.float32)
    res[idx] = val
    return res
