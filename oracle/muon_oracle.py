"""fp64 CPU oracle: Muon step (momentum -> Frobenius normalisation ->
Newton-Schulz -> scaled apply with decoupled weight decay) and AdamW step.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use this module. It shares no code with the HIP path:
it imports only NumPy.

Sources, cited by page title and section:

[OPT]  "Optimizer tutorial" page on mhpq.cn (large-model training series,
       part 2: from SGD to Adam, AdamW and Muon).  Its numbered sections:
       2.1 Momentum, 2.3 Adam, 2.4 Adam's memory cost, 3.1 Adam vs AdamW,
       3.3 optimizer state under mixed precision, 4.2 Newton-Schulz
       iteration, 4.3 Muon + Adam in practice.
[K2]   Zhihu answer by toothacher17 on the Kimi K2 release.  Sections
       2.1 Zero-1 sharding, 2.2 Moonshot's solution, 3.1 Standard
       parametrisation + Muon, 3.2 MuP parametrisation + Muon,
       4 Concern 3 (training instabilities).

Everything is computed in float64.  Only the *_stored wrappers round, once,
at the end of a step, to the storage precision of each buffer (fp32 states,
bf16 or fp32 params), so that multi-step runs see the same storage
precision as the GPU.

Readings taken where the pages are silent, garbled or loose (each is also
listed with its reason in the design notes of the repository):

R1  Momentum is the EMA printed in [OPT] 2.1: M <- mu*M + (1-mu)*G.
R2  Nesterov look-ahead (not on the pages): U = mu*M_new + (1-mu)*G.
    Without Nesterov, U = M_new.
R3  Newton-Schulz acts on the momentum look-ahead U, after Frobenius
    normalisation X0 = U / (||U||_F + eps)  ([K2] 4 gives
    ||.||_2 <= ||.||_F, so sigma_max(X0) <= 1).
R4  The NS step is X <- a*X + (b*A + c*A@A) @ X with A = X @ X^T.  [OPT] 4.2
    prints the cubic (a, b, c) = (3/2, -1/2, 0); any (a, b, c) is accepted.
R5  Tall matrices (rows > cols) are iterated in transposed form so that the
    Gram matrix is min(r,c) square; the odd matrix polynomial commutes with
    transposition, so the result is identical in exact arithmetic.
R6  Update scale s (mode 0): rms_target * sqrt(max(r, c)), which makes the
    RMS of s*O equal rms_target when O is orthogonal ([K2] 3.1: Muon's
    update RMS is matched to AdamW's 0.2-0.4).  Mode 1:
    sqrt(max(1, rows/cols)) ([K2] 3.2, d_out = rows of an [out, in]
    weight).  Mode 2: s = 1.
R7  Muon weight decay is decoupled, as in [OPT] 3.1, and uses the old W:
    W <- W - lr*wd*W - lr*s*O.
R8  AdamW as printed in [OPT] 2.3 and 3.1 with the extraction damage undone:
    theta <- theta - lr*m_hat/(sqrt(v_hat) + eps) - lr*wd*theta_old,
    eps outside the square root, t starting at 1.
R9  Mixed precision ([OPT] 3.3): the update runs on the fp32 master copy and
    the bf16 parameter is the round-to-nearest-even cast of that fp32 value.
R13 Compressed AdamW states ([OPT] 2.4 lists 8-bit AdamW states; 3.3: v
    tolerates FP16 or 8-bit storage, m is more sensitive, so v is compressed
    first): a step reads m and v from their storage type, computes in full
    precision, and stores m as fp32 or bf16 and v as fp32, bf16 or fp16
    (round to nearest even).  The pages fix no 8-bit encoding; none is
    defined here.

Parity status: every function below is pinned by tests/test_oracle_pins.py
(closed forms, SVD spectral calculus, invariants, library bf16 casts).
The readings R2, R5 (beyond exact invariance), R6 mode 1 and the default
rms_target 0.2 come from this document's readings, not from printed values.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# storage rounding ([OPT] 3.3: fp32 master, cast back to 16 bit)
# --------------------------------------------------------------------------


def fp32_round(x) -> np.ndarray:
    """Round float64 values to the nearest float32 (IEEE RNE), back as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round to bfloat16 (round-to-nearest-even on the fp32 bit pattern).

    The input is first rounded to fp32 (that is the value a fp32 master
    copy holds, reading R9); the low 16 bits are then rounded away with
    ties to even.  NaN stays NaN.  Returned as float64 holding the
    bf16 value exactly.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) >> 16
    out_bits = (rounded << 16).astype(np.uint32)
    out = out_bits.view(np.float32).astype(np.float64)
    nan = np.isnan(f)
    if np.any(nan):
        out = np.where(nan, np.nan, out)
    return out


def fp16_round(x) -> np.ndarray:
    """Round to IEEE binary16 (round to nearest even; subnormals kept;
    beyond the largest finite value, +-inf).  As for bf16, the input is first
    rounded to fp32, the precision the step computes in.  Returned as
    float64 holding the fp16 value exactly."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16).astype(
            np.float64)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "fp16":
        return fp16_round(x)
    if dtype == "fp32":
        return fp32_round(x)
    if dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# hyperparameters
# --------------------------------------------------------------------------


@dataclasses.dataclass
class MuonHP:
    lr: float = 0.02
    weight_decay: float = 0.1
    momentum: float = 0.95
    nesterov: bool = True
    ns_a: float = 1.5
    ns_b: float = -0.5
    ns_c: float = 0.0
    ns_steps: int = 5
    eps: float = 1e-7
    scale_mode: int = 0
    rms_target: float = 0.2


@dataclasses.dataclass
class AdamWHP:
    lr: float = 0.02
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1


# --------------------------------------------------------------------------
# Muon pieces
# --------------------------------------------------------------------------


def ema_momentum(M: np.ndarray, G: np.ndarray, mu: float) -> np.ndarray:
    """[OPT] 2.1: the momentum buffer is an exponential moving average of
    the gradient, M_new = mu*M + (1-mu)*G (reading R1)."""
    return mu * M + (1.0 - mu) * G


def nesterov_lookahead(M_new: np.ndarray, G: np.ndarray, mu: float,
                       nesterov: bool) -> np.ndarray:
    """Reading R2: the matrix handed to Newton-Schulz.  With Nesterov it is
    the look-ahead mu*M_new + (1-mu)*G, otherwise M_new itself."""
    if nesterov:
        return mu * M_new + (1.0 - mu) * G
    return M_new


def frobenius_normalise(U: np.ndarray, eps: float) -> np.ndarray:
    """Reading R3 ([K2] 4: spectral norm <= Frobenius norm): divide by
    ||U||_F + eps so that every singular value of the result is <= 1."""
    return U / (np.linalg.norm(U) + eps)


def ns_iteration(X: np.ndarray, a: float, b: float, c: float) -> np.ndarray:
    """One Newton-Schulz step, [OPT] 4.2 (reading R4):
    A = X X^T, B = b*A + c*A A, X_next = a*X + B X.
    With (a, b, c) = (3/2, -1/2, 0) this is the printed (3X - X X^T X)/2."""
    A = X @ X.T
    B = b * A
    if c != 0.0:
        B = B + c * (A @ A)
    return a * X + B @ X


def newton_schulz(X0: np.ndarray, a: float, b: float, c: float,
                  steps: int) -> np.ndarray:
    """Run ``steps`` NS iterations on X0 ([OPT] 4.2: a fixed count, typically
    5).  Tall inputs are iterated in transposed form (reading R5)."""
    tall = X0.shape[0] > X0.shape[1]
    X = X0.T if tall else X0
    for _ in range(steps):
        X = ns_iteration(X, a, b, c)
    return X.T if tall else X


def update_scale(rows: int, cols: int, mode: int, rms_target: float) -> float:
    """Per-matrix update multiplier s (reading R6).

    mode 0: rms_target*sqrt(max(r, c))  ([K2] 3.1, update-RMS matching)
    mode 1: sqrt(max(1, rows/cols))     ([K2] 3.2, max(1, sqrt(d_out/d_in)))
    mode 2: 1
    """
    if mode == 0:
        return rms_target * math.sqrt(max(rows, cols))
    if mode == 1:
        return math.sqrt(max(1.0, rows / cols))
    if mode == 2:
        return 1.0
    raise ValueError(f"unknown scale mode {mode}")


def muon_matrix_math(W: np.ndarray, G: np.ndarray, M: np.ndarray,
                     hp: MuonHP, grad_scale: float = 1.0
                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Muon step for one matrix, in fp64, no storage rounding.

    Returns (W_new, M_new, O) where O is the orthogonalised update.
    The order (momentum, normalise, NS, apply) is reading R3 / R7.
    ``grad_scale`` multiplies the gradient first (the clip factor of a
    clipped step, oracle/guard_oracle.py reading G2).
    """
    W = np.asarray(W, dtype=np.float64)
    G = grad_scale * np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    rows, cols = W.shape
    M_new = ema_momentum(M, G, hp.momentum)
    U = nesterov_lookahead(M_new, G, hp.momentum, hp.nesterov)
    X0 = frobenius_normalise(U, hp.eps)
    O = newton_schulz(X0, hp.ns_a, hp.ns_b, hp.ns_c, hp.ns_steps)
    s = update_scale(rows, cols, hp.scale_mode, hp.rms_target)
    W_new = W - hp.lr * hp.weight_decay * W - hp.lr * s * O
    return W_new, M_new, O


def muon_step_flat(params: np.ndarray, grads: np.ndarray, momentum: np.ndarray,
                   mats: Sequence[Tuple[int, int, int]], hp: MuonHP,
                   param_dtype: str, only: Sequence[int] | None = None,
                   grad_scale: float = 1.0
                   ) -> Tuple[np.ndarray, np.ndarray, Dict[int, np.ndarray]]:
    """Muon step over a flat concatenated buffer ([K2] 2.2: all parameters
    flattened and concatenated; each matrix addressed by its element offset).

    ``mats`` holds (offset, rows, cols) per matrix, row-major.  Elements not
    covered by a matrix are left untouched.  ``only`` restricts the work to
    the listed matrix indices (sampled parity at large sizes).
    ``grad_scale`` multiplies every gradient (a clipped step).
    Returns (params_new, momentum_new, {index: O}) with params rounded to
    ``param_dtype`` and momentum to fp32, once, at the end of the step.
    """
    p = np.array(params, dtype=np.float64, copy=True)
    mom = np.array(momentum, dtype=np.float64, copy=True)
    g = np.asarray(grads, dtype=np.float64)
    outs: Dict[int, np.ndarray] = {}
    idx = range(len(mats)) if only is None else only
    for i in idx:
        off, r, c = mats[i]
        sl = slice(off, off + r * c)
        W_new, M_new, O = muon_matrix_math(p[sl].reshape(r, c),
                                           g[sl].reshape(r, c),
                                           mom[sl].reshape(r, c), hp, grad_scale)
        p[sl] = round_to(W_new, param_dtype).reshape(-1)
        mom[sl] = fp32_round(M_new).reshape(-1)
        outs[i] = O
    return p, mom, outs


def ns_flops(rows: int, cols: int, steps: int, c: float) -> float:
    """Algorithmic flops of the NS iterations on one matrix: per step
    m(m+1)n for the symmetric X X^T (one triangle), m^2(m+1) for the
    symmetric A A when c != 0, and 2 m^2 n for B X; m = min, n = max."""
    m, n = min(rows, cols), max(rows, cols)
    per = m * (m + 1) * n + 2 * m * m * n
    if c != 0.0:
        per += m * m * (m + 1)
    return float(per) * steps


# --------------------------------------------------------------------------
# AdamW ([OPT] 2.3 Adam, 3.1 AdamW decoupled weight decay)
# --------------------------------------------------------------------------


def adamw_math(theta: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray,
               hp: AdamWHP, t: int, grad_scale: float = 1.0
               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One AdamW step in fp64, as printed (reading R8).  t >= 1.

    m <- b1 m + (1-b1) g ; v <- b2 v + (1-b2) g^2
    m_hat = m/(1-b1^t) ; v_hat = v/(1-b2^t)
    theta <- theta - lr*m_hat/(sqrt(v_hat)+eps) - lr*wd*theta_old
    ``grad_scale`` multiplies g first (a clipped step).
    """
    if t < 1:
        raise ValueError("AdamW step count starts at 1")
    theta = np.asarray(theta, dtype=np.float64)
    g = grad_scale * np.asarray(g, dtype=np.float64)
    m_new = hp.beta1 * np.asarray(m, dtype=np.float64) + (1.0 - hp.beta1) * g
    v_new = hp.beta2 * np.asarray(v, dtype=np.float64) + (1.0 - hp.beta2) * g * g
    m_hat = m_new / (1.0 - hp.beta1 ** t)
    v_hat = v_new / (1.0 - hp.beta2 ** t)
    theta_new = (theta - hp.lr * m_hat / (np.sqrt(v_hat) + hp.eps)
                 - hp.lr * hp.weight_decay * theta)
    return theta_new, m_new, v_new


def adamw_step_stored(param: np.ndarray, master: np.ndarray | None,
                      g: np.ndarray, m: np.ndarray, v: np.ndarray,
                      hp: AdamWHP, t: int, param_dtype: str, grad_scale: float = 1.0,
                      m_dtype: str = "fp32", v_dtype: str = "fp32"
                      ) -> Tuple[np.ndarray, np.ndarray | None, np.ndarray, np.ndarray]:
    """AdamW step with storage rounding ([OPT] 3.3, readings R9, R13).

    With a master copy: the fp32 master is updated and the parameter becomes
    the bf16 (or fp32) cast of the new fp32 master.  Without one: the
    parameter itself must be fp32 and is updated in place.  m and v are
    stored as ``m_dtype`` / ``v_dtype`` (their inputs are the stored values
    of the previous step).
    Returns (param_new, master_new or None, m_new, v_new).
    """
    theta = master if master is not None else param
    th, m_new, v_new = adamw_math(theta, g, m, v, hp, t, grad_scale)
    th32 = fp32_round(th)
    m_st, v_st = round_to(m_new, m_dtype), round_to(v_new, v_dtype)
    if master is not None:
        return round_to(th32, param_dtype), th32, m_st, v_st
    if param_dtype != "fp32":
        raise ValueError("without a master copy the parameter must be fp32")
    return th32, None, m_st, v_st


def adamw_state_bytes_per_param(m_dtype: str = "fp32", v_dtype: str = "fp32") -> int:
    """[OPT] 2.4: Adam keeps two states per parameter, fp32 in the standard
    implementation (8 bytes); compressed states take their storage size."""
    size = {"fp32": 4, "bf16": 2, "fp16": 2}
    return size[m_dtype] + size[v_dtype]


def muon_state_bytes_per_param() -> int:
    """[OPT] 4.3: Muon keeps one fp32 state buffer where Adam keeps two."""
    return 4


__all__: List[str] = [
    "AdamWHP", "MuonHP", "adamw_math", "adamw_state_bytes_per_param", "adamw_step_stored",
    "bf16_round", "fp16_round",
    "ema_momentum", "fp32_round", "frobenius_normalise", "muon_matrix_math",
    "muon_step_flat", "nesterov_lookahead", "newton_schulz", "ns_flops",
    "ns_iteration", "round_to", "update_scale",
]
