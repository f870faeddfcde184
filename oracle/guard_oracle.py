"""fp64 CPU oracle for the safety net around the optimizer step: global
gradient-norm clipping, the non-finite guard that skips a step, and
optimizer-state statistics.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use this module. It shares no code with the HIP path:
it imports only NumPy.

Source, cited by page title and section:

[OPT]  "Optimizer tutorial" page on mhpq.cn (large-model training series,
       part 2), section 5.4 (optimizer numerical faults under mixed
       precision and how to track them down) and the practical notes that
       close the page:
         - when NaN appears, look first at whether m and v hold Inf, then at
           whether the gradient after clip_grad_norm is still abnormal;
         - frameworks put an "Inf guard" on the optimizer state that skips
           the current step when it detects an anomaly;
         - keep gradient clipping as a safety net even with Adam, with a
           larger threshold on large models (max_grad_norm 1.0 is
           conservative there; 2.0 or 5.0 can suit better);
         - log statistics of the optimizer state (the mean and variance of
           m): v dropping by orders of magnitude announces vanishing
           gradients, extreme values in m an abnormal gradient step.

Readings where the page is silent:

G1  The clipping norm is the global L2 norm over every gradient element of
    every parameter (Muon matrices and AdamW parameters alike), accumulated
    in fp64: norm = sqrt(sum g^2).
G2  Clip factor f = min(1, max_norm / (norm + eps)) with eps = 1e-6 by
    default, applied as g <- f * g before the step: momentum and AdamW see
    the scaled gradient.  max_norm <= 0 disables clipping (f = 1).
G3  Guard: the whole step is skipped (parameters and every state buffer
    unchanged) when the global norm is not finite, i.e. when any gradient
    element is NaN or +-Inf.
G4  Statistics of a state buffer: count, mean, population variance, min,
    max and max |x| over its finite elements, and the count of non-finite
    elements (NaN, +-Inf).  Over no finite element the six values are 0.

Parity status: every function is pinned by tests/test_oracle_guard_pins.py
(closed forms: constant buffers, a 3-4-5 norm, arithmetic sequences; the
scale invariance of Muon's normalised update; the closed-form first AdamW
step).  G1, G2's eps and G4's treatment of non-finite elements are this
module's readings, not printed values.
"""

from __future__ import annotations

import math
from typing import Dict, Sequence

import numpy as np

CLIP_EPS = 1e-6


def global_grad_norm(buffers: Sequence[np.ndarray]) -> float:
    """Reading G1: sqrt of the sum of squares of every element of every
    buffer, in fp64 (NaN or Inf anywhere gives a non-finite norm)."""
    total = 0.0
    for b in buffers:
        x = np.asarray(b, dtype=np.float64).reshape(-1)
        total += float(np.dot(x, x))
    return math.sqrt(total) if total >= 0.0 else float("nan")


def guard_skip(norm: float) -> bool:
    """Reading G3: skip the step when the global gradient norm is not finite."""
    return not math.isfinite(norm)


def clip_factor(norm: float, max_norm: float, eps: float = CLIP_EPS) -> float:
    """Reading G2: the factor the gradients are multiplied by before the step
    (1 when clipping is off, the norm is within max_norm, or the step is
    skipped anyway)."""
    if max_norm <= 0.0 or guard_skip(norm):
        return 1.0
    return min(1.0, max_norm / (norm + eps))


def state_stats(x: np.ndarray) -> Dict[str, float]:
    """Reading G4: statistics of one optimizer-state buffer."""
    v = np.asarray(x, dtype=np.float64).reshape(-1)
    finite = np.isfinite(v)
    f = v[finite]
    out = {"count": int(f.size), "nonfinite": int(v.size - f.size),
           "mean": 0.0, "var": 0.0, "min": 0.0, "max": 0.0, "absmax": 0.0}
    if f.size:
        mean = float(np.mean(f))
        out.update(mean=mean, var=float(np.mean((f - mean) ** 2)), min=float(f.min()),
                   max=float(f.max()), absmax=float(np.max(np.abs(f))))
    return out


__all__ = ["CLIP_EPS", "clip_factor", "global_grad_norm", "guard_skip", "state_stats"]
