"""Accordion's two-level switch (oracle, test infrastructure).

Source: "Accordion: Adaptive Gradient Communication via Critical Learning
Regime Identification", method section: the rate of change of the
gradient-norm magnitude marks critical regimes; inside one the compressor uses
the low-compression level l_low (e.g. PowerSGD rank 2 instead of rank 1, or a
larger K for top-k), outside it the high-compression level l_high.  The results
section reports the norm-change rate as a reliable indicator.

The pages print no formula.  Readings taken:
  * per layer l, at a check step:  rho = |N_prev - N_now| / N_prev
    (N_prev = 0: rho = +inf if N_now > 0, else 0);
  * critical (l_low) when rho >= threshold, otherwise l_high;
  * no previous check -> l_low (nothing known yet: the safe, low-compression level);
  * N_prev <- N_now after every check.
The comparison is made in float64 from the float32 norms.
"""
from __future__ import annotations

import numpy as np

LEVEL_LOW = 0    # l_low: low compression, used in critical regimes
LEVEL_HIGH = 1   # l_high: high compression


def accordion_select(norm_now, norm_prev, has_prev: bool, threshold: float):
    """Return (levels, new_prev) for one check over all layers."""
    now = np.asarray(norm_now, np.float32).astype(np.float64)
    prev = np.asarray(norm_prev, np.float32).astype(np.float64)
    thr = float(np.float32(threshold))
    levels = np.empty(now.size, np.int32)
    for l in range(now.size):
        if not has_prev:
            levels[l] = LEVEL_LOW
            continue
        if prev[l] == 0.0:
            rho = np.inf if now[l] > 0.0 else 0.0
        else:
            rho = abs(prev[l] - now[l]) / prev[l]
        levels[l] = LEVEL_LOW if rho >= thr else LEVEL_HIGH
    return levels, np.asarray(norm_now, np.float32).copy()
