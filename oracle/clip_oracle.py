"""fp64 CPU oracle for MuonClip: a scalar rescale of attention projection
weights (W_q, W_k, whole matrices or one head's block of rows) after the
optimizer step, to keep attention logits bounded.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use this module. It shares no code with the HIP path:
it imports only NumPy and the storage-rounding helpers of the Muon oracle.

Source, cited by page title and section:

[K2]  Zhihu answer by toothacher17 on the Kimi K2 release, section 4
      ("Muon training instabilities", the MuonClip part): the max attention
      logit grows in large Muon runs; QK-norm cannot be used with MLA since
      the per-head q and k are never materialised; the spectral norm is at
      most the Frobenius norm and bounds ||xW||_2 <= ||x||_2 ||W||_2, so the
      answer's author reads MuonClip as a clip on the Frobenius norm of the
      weight, which controls ||xW||_2; the method's author, asked, said the
      idea is rather to act directly on the root problem, the max logit.

Readings where the page is silent:

MC1 Frobenius mode (the mechanism the page spells out).  For each target
    block W: gamma = min(1, tau / ||W||_F), W <- gamma * W.  Afterwards
    ||W||_2 <= ||W||_F <= tau, so ||x W^T||_2 <= tau ||x||_2 for every row
    vector x.  gamma = 1 when ||W||_F is 0 or not finite.
MC2 Max-logit mode (acting on the logit itself).  The caller supplies, per
    group g, the largest attention logit S_g seen in the forward pass (one
    head, or one layer).  When S_g > tau, every block of that group (that
    head's W_q and W_k rows) is multiplied by gamma = sqrt(tau / S_g): a
    logit q . k is bilinear in (W_q, W_k), so it scales by gamma^2 and the
    largest becomes exactly tau.  The even split of the factor between W_q
    and W_k is this reading's choice; the page gives no formula.
    gamma = 1 when S_g <= tau or S_g is not finite.
MC3 A target block is rows x cols elements of the flat parameter buffer,
    element (r, c) at offset + r * ld + c (ld >= cols): a whole [out, in]
    row-major matrix (ld = cols), or one head's block of rows of it.
    Blocks do not overlap.  Elements outside every block are untouched.
MC4 The new value is rounded to the parameter's storage type (bf16 RNE or
    fp32) once, from gamma * w in fp64.

Parity status: every function is pinned by tests/test_oracle_clip_pins.py
(closed forms: a diag(3, 4) matrix, rank-one blocks where the spectral and
Frobenius norms coincide; the spectral bound through an SVD; the max logit
of a small attention head recomputed after the clip equals tau; untouched
elements and heads).  MC2's even split and the non-finite rules are this
module's readings, not printed values.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

from oracle.muon_oracle import round_to

MODE_FROBENIUS = 0
MODE_MAX_LOGIT = 1


def frobenius_clip_factor(block: np.ndarray, tau: float) -> Tuple[float, float]:
    """Reading MC1: (||W||_F, gamma) for one block."""
    w = np.asarray(block, dtype=np.float64).reshape(-1)
    norm = math.sqrt(float(np.dot(w, w)))
    if not math.isfinite(norm) or norm <= tau or norm == 0.0:
        return norm, 1.0
    return norm, tau / norm


def logit_clip_factor(max_logit: float, tau: float) -> float:
    """Reading MC2: gamma for every block of a group whose largest logit is
    ``max_logit``."""
    if not math.isfinite(max_logit) or max_logit <= tau:
        return 1.0
    return math.sqrt(tau / max_logit)


def block_view(flat: np.ndarray, target) -> Tuple[np.ndarray, np.ndarray]:
    """Reading MC3: the flat indices of a target block, as a rows x cols
    array, and the block's values (fp64)."""
    offset, rows, cols, ld = target[0], target[1], target[2], target[3]
    idx = offset + np.arange(rows)[:, None] * ld + np.arange(cols)[None, :]
    return idx, np.asarray(flat, dtype=np.float64)[idx]


def muon_clip_flat(params: np.ndarray, targets: Sequence, mode: int, tau: float,
                   max_logits: Sequence[float] | None, param_dtype: str
                   ) -> Tuple[np.ndarray, List[float], List[float]]:
    """MuonClip over the flat parameter buffer.

    targets: (offset, rows, cols, ld, group) per block.  Returns the new
    flat buffer (rounded to ``param_dtype``, reading MC4), and per target
    the Frobenius norm before the clip (0 in max-logit mode) and gamma.
    """
    if not (tau > 0.0 and math.isfinite(tau)):
        raise ValueError("tau must be finite and > 0")
    out = np.asarray(params, dtype=np.float64).copy()
    norms, gammas = [], []
    for t in targets:
        idx, w = block_view(params, t)
        if mode == MODE_FROBENIUS:
            norm, gamma = frobenius_clip_factor(w, tau)
        elif mode == MODE_MAX_LOGIT:
            norm, gamma = 0.0, logit_clip_factor(float(max_logits[t[4]]), tau)
        else:
            raise ValueError("unknown mode")
        norms.append(norm)
        gammas.append(gamma)
        if gamma != 1.0:
            out[idx] = round_to(gamma * w, param_dtype)
    return out, norms, gammas


def attention_max_logit(x: np.ndarray, wq_head: np.ndarray, wk_head: np.ndarray) -> float:
    """Largest logit of one attention head: max over query and key rows
    i, j of (x_i W_q^T) . (x_j W_k^T), with W_q, W_k the head's
    [d_head, d_model] blocks (a logit's 1/sqrt(d_head) factor is left out:
    a constant does not change where the threshold bites)."""
    q = np.asarray(x, np.float64) @ np.asarray(wq_head, np.float64).T
    k = np.asarray(x, np.float64) @ np.asarray(wk_head, np.float64).T
    return float(np.max(q @ k.T))


__all__ = ["MODE_FROBENIUS", "MODE_MAX_LOGIT", "attention_max_logit", "block_view",
           "frobenius_clip_factor", "logit_clip_factor", "muon_clip_flat"]
