"""CPU oracle for the gradient-compressor hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy code, float64 wherever the pages leave the
precision open.  It is the reference that the HIP path is checked against and
shares no code with it (no common kernels, helpers, tables or constants).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never calls it.

Sources (the three review pages):
  * "Sparsified SGD with Memory" (Stich, Cordonnier, Jaggi) -- method section:
    the memory update of Mem-SGD, the k-contraction operators (top-k, rand-k),
    the step size eta_t = 8/(mu(a+t)); abstract: the most significant entries
    (top-k).
  * "Accordion: Adaptive Gradient Communication via Critical Learning Regime
    Identification" -- method section: two compression levels l_low / l_high
    chosen from the rate of change of the gradient norm; works with PowerSGD
    rank r and top-k.
  * "On the Utility of Gradient Compression in Distributed Training Systems" --
    method/results sections: PowerSGD as the all-reduce compatible compressor
    whose encode/decode time is the cost being measured.

PowerSGD's individual steps (P = M Q, orthonormalise P, Q = M^T P, decode
P Q^T, residual into memory) are not spelled out on the pages; the oracle takes
them in that plain order (see ``powersgd.py``).  The vectors of a gradient set
(batch-norm parameters, biases) are sent uncompressed (``passthrough.py``).

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against closed forms, brute force, library special cases or invariants fixed by
the pages.  ``memsgd.run_memsgd`` is pinned only qualitatively (convergence at
the SGD rate) -- parity unpinned beyond that claim.
"""
from .topk_ef import (ef_accumulate, grad_to_f64, topk_select, topk_ef_step,
                      topk_decode, magnitude_order)
from .randk_ef import randk_ef_step
from .powersgd import orthonormalize_mgs, powersgd_ef_step
from .passthrough import passthrough_step
from .norms import grad_norm
from .accordion import accordion_select, LEVEL_LOW, LEVEL_HIGH
from .memsgd import run_memsgd, QuadraticProblem

__all__ = [
    "ef_accumulate", "grad_to_f64", "topk_select", "topk_ef_step", "topk_decode",
    "magnitude_order", "randk_ef_step", "orthonormalize_mgs", "powersgd_ef_step", "passthrough_step", "grad_norm",
    "accordion_select", "LEVEL_LOW", "LEVEL_HIGH", "run_memsgd", "QuadraticProblem",
]
