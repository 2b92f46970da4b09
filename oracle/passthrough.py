"""Tensors sent uncompressed (oracle, test infrastructure).

A gradient set holds weight matrices, which the low-rank compressor takes
(Accordion paper, method section: PowerSGD on the layers of ResNet-18 and
VGG-19), and small vectors -- batch-norm scales and shifts, biases -- that are
sent as they are.  Their step is the plain scaled gradient

    out = eta * grad,   memory untouched (nothing is left out)

Reading: one float32 rounding of the exact product, with eta used as a float32
value (as in the error-feedback accumulate).  The product of two float32
numbers is exact in float64, so rounding that once gives the correctly rounded
float32 product.
"""
from __future__ import annotations

import numpy as np

from .topk_ef import grad_to_f64


def passthrough_step(grad: np.ndarray, eta: float) -> np.ndarray:
    """out = fl32(eta * grad) for one vector (float32, or bf16 bits as uint16)."""
    eta64 = np.float64(np.float32(eta))
    return (eta64 * grad_to_f64(np.asarray(grad).ravel())).astype(np.float32)
