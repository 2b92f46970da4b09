"""Per-layer gradient norm (oracle, test infrastructure).

Accordion (method section) detects critical regimes from how fast the
magnitude of the gradient norm changes; the norm is the Euclidean norm of a
layer's gradient.  Reading: the raw gradient of the step, as stored (float32
or bf16), before any error-feedback accumulation.

Squares of float32/bf16 values are exact in float64; ``math.fsum`` returns the
correctly rounded sum; the square root is taken once at the end.
"""
from __future__ import annotations

import math

import numpy as np

from .topk_ef import grad_to_f64


def grad_norm(grad: np.ndarray) -> float:
    g = grad_to_f64(np.asarray(grad).ravel())
    return math.sqrt(math.fsum(g * g))
