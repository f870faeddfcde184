"""Workload definitions and seeded synthetic input generators.

This module holds no optimizer arithmetic: it only describes shapes,
storage dtypes, hyperparameter values and value distributions, and draws
seeded random tensors.  Both the HIP path (through the binding) and the
fp64 oracle (in the tests and the bench's CPU baseline) take their inputs
from here.

Workloads (rows x cols are the matrix as the caller stores it, row-major):

* ``single_fp32_128x256``  one fp32 128x256 matrix, W and G ~ N(0,1), zero
  momentum, mu 0.95 Nesterov, 5 NS steps, lr 0.02, wd 0.1; plus a fp32
  vector of 4096 params under AdamW (b1 0.9, b2 0.95, eps 1e-8), 10 steps.
* ``dense_d2048_l16``  16 transformer layers, d = 2048: Wq/Wk/Wv/Wo 2048x2048,
  gate/up 2048x5632, down 5632x2048 in bf16 (N(0, 0.02^2)), fp32 momentum;
  embedding and LM head 32000x2048 and 33 RMSNorm vectors of 2048 under
  AdamW with bf16 params/grads and fp32 master, m, v.
* ``moe_e64_2048x1408``  64 experts x (gate, up 2048x1408; down 1408x2048),
  packed as [E, H, H'] blocks; G ~ N(0, 1e-4^2), W ~ N(0, 0.006^2).
* ``moe_e384_7168x2048``  384 experts x (gate, up 7168x2048; down
  2048x7168), G std 1e-4, W std 0.006 (1152 matrices, 1.69e10 params);
  ``moe_e128_7168x2048`` is the 128-expert share (5.6e9 params).
* ``ragged_500``  500 matrices with dims drawn from 64*{8..128}, square, tall
  and wide, every tenth with dims off the 64 grid; plus a 163840x7168
  embedding and 128 vectors of 7168 under AdamW with fp32 master.

The expert layout follows the MoonEP news item ("memory contract": one
contiguous [E, H, H'] weight tensor per projection, experts addressed by
row offset).
"""

from __future__ import annotations

import dataclasses
import json
import math
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

# tensor kinds used in the seed key
KIND_W, KIND_G, KIND_ADAM_P, KIND_ADAM_G = 0, 1, 2, 3

CUBIC = (1.5, -0.5, 0.0)          # the optimizer tutorial's printed iteration
QUINTIC = (15.0 / 8.0, -5.0 / 4.0, 3.0 / 8.0)


@dataclasses.dataclass
class MuonHParams:
    lr: float = 0.02
    weight_decay: float = 0.1
    momentum: float = 0.95
    nesterov: bool = True
    ns_a: float = CUBIC[0]
    ns_b: float = CUBIC[1]
    ns_c: float = CUBIC[2]
    ns_steps: int = 5
    eps: float = 1e-7
    scale_mode: int = 0
    rms_target: float = 0.2


@dataclasses.dataclass
class AdamWHParams:
    lr: float = 0.02
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1


@dataclasses.dataclass
class AdamGroup:
    name: str
    numel: int
    param_dtype: str          # "bf16" or "fp32"
    grad_dtype: str
    master: bool              # fp32 master copy present
    p_std: float
    g_std: float
    p_const: Optional[float] = None   # e.g. RMSNorm gamma = 1


@dataclasses.dataclass
class Workload:
    name: str
    config_id: int
    shapes: List[Tuple[int, int]]
    param_dtype: str
    grad_dtype: str
    w_std: float
    g_std: float
    adam: List[AdamGroup]
    muon_hp: MuonHParams
    adam_hp: AdamWHParams
    steps: int = 1            # consecutive optimizer steps the workload names

    # flat layout: matrices concatenated in order
    def offsets(self) -> List[int]:
        offs, o = [], 0
        for r, c in self.shapes:
            offs.append(o)
            o += r * c
        return offs

    def mats(self) -> List[Tuple[int, int, int]]:
        return [(o, r, c) for o, (r, c) in zip(self.offsets(), self.shapes)]

    def muon_numel(self) -> int:
        return sum(r * c for r, c in self.shapes)

    def adam_numel(self) -> int:
        return sum(g.numel for g in self.adam)


def _dense_shapes(d: int, ff: int, layers: int) -> List[Tuple[int, int]]:
    out = []
    for _ in range(layers):
        out += [(d, d)] * 4           # Wq, Wk, Wv, Wo
        out += [(d, ff), (d, ff)]     # gate, up
        out += [(ff, d)]              # down
    return out


def _moe_shapes(experts: int, h: int, hp: int) -> List[Tuple[int, int]]:
    # gate [E, H, H'] || up [E, H, H'] || down [E, H', H]
    return [(h, hp)] * experts + [(h, hp)] * experts + [(hp, h)] * experts


def ragged_shapes(count: int = 500, seed: int = 5) -> List[Tuple[int, int]]:
    """Seeded ragged shape draw: dims 64*U{8..128}; i mod 3 picks square,
    tall or wide; every tenth matrix gets U{1..63} added to each dim
    (clamped to 8192) so its dims leave the 64 grid."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0])))
    out = []
    for i in range(count):
        d1 = 64 * int(rng.integers(8, 129))
        d2 = 64 * int(rng.integers(8, 129))
        if i % 10 == 0:
            d1 = min(8192, d1 + int(rng.integers(1, 64)))
            d2 = min(8192, d2 + int(rng.integers(1, 64)))
        kind = i % 3
        if kind == 0:
            r = c = d1
        elif kind == 1:
            r, c = max(d1, d2), min(d1, d2)
        else:
            r, c = min(d1, d2), max(d1, d2)
        out.append((r, c))
    return out


RAGGED_500_JSON = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                               "ragged_500_shapes.json")


def frozen_ragged_shapes(path: str = RAGGED_500_JSON) -> List[Tuple[int, int]]:
    """The ragged workload's shape list as committed (written once by
    ``python -m muon_newton_schulz_amd.workloads --freeze-ragged`` from
    ragged_shapes()), so that every run, test and profile sees the same
    matrices whatever the NumPy version."""
    with open(path) as f:
        data = json.load(f)
    return [(int(r), int(c)) for r, c in data["shapes"]]


def write_frozen_ragged_shapes(path: str = RAGGED_500_JSON) -> None:
    shapes = ragged_shapes()
    data = {"recipe": "ragged_shapes(count=500, seed=5): NumPy PCG64 seeded with "
                      "SeedSequence([5, 0]); per matrix i: d1, d2 = 64*U{8..128}; for i % 10 "
                      "== 0 each dim + U{1..63}, clamped to 8192; i % 3 = 0 square (d1 x d1), "
                      "1 tall (max x min), 2 wide (min x max)",
            "count": len(shapes), "params": sum(r * c for r, c in shapes),
            "shapes": [[r, c] for r, c in shapes]}
    with open(path, "w") as f:
        json.dump(data, f, separators=(",", ":"))
        f.write("\n")


def workload(name: str) -> Workload:
    mhp = MuonHParams()
    ahp = AdamWHParams()
    if name == "single_fp32_128x256":
        return Workload(name, 1, [(128, 256)], "fp32", "fp32", 1.0, 1.0,
                        [AdamGroup("vector4096", 4096, "fp32", "fp32", False, 1.0, 1.0)],
                        mhp, ahp, steps=10)
    if name == "dense_d2048_l16":
        d, ff, L, vocab = 2048, 5632, 16, 32000
        adam = [AdamGroup("embedding", vocab * d, "bf16", "bf16", True, 0.02, 0.02),
                AdamGroup("lm_head", vocab * d, "bf16", "bf16", True, 0.02, 0.02),
                AdamGroup("rmsnorm", (2 * L + 1) * d, "bf16", "bf16", True, 0.0, 0.02,
                          p_const=1.0)]
        return Workload(name, 2, _dense_shapes(d, ff, L), "bf16", "bf16", 0.02, 0.02,
                        adam, mhp, ahp)
    if name == "moe_e64_2048x1408":
        return Workload(name, 3, _moe_shapes(64, 2048, 1408), "bf16", "bf16", 0.006, 1e-4,
                        [], mhp, ahp)
    if name == "moe_e384_7168x2048":
        return Workload(name, 4, _moe_shapes(384, 7168, 2048), "bf16", "bf16", 0.006, 1e-4,
                        [], mhp, ahp)
    if name == "moe_e128_7168x2048":
        return Workload(name, 4, _moe_shapes(128, 7168, 2048), "bf16", "bf16", 0.006, 1e-4,
                        [], mhp, ahp)
    if name == "ragged_500":
        adam = [AdamGroup("embedding", 163840 * 7168, "bf16", "bf16", True, 0.02, 0.02),
                AdamGroup("vectors", 128 * 7168, "bf16", "bf16", True, 0.0, 0.02,
                          p_const=1.0)]
        return Workload(name, 5, frozen_ragged_shapes(), "bf16", "bf16", 0.02, 0.02, adam,
                        mhp, ahp)
    raise KeyError(name)


WORKLOADS = ["single_fp32_128x256", "dense_d2048_l16", "moe_e64_2048x1408",
             "moe_e384_7168x2048", "moe_e128_7168x2048", "ragged_500"]

# --------------------------------------------------------------------------
# seeded generation
# --------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _M64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def seed_key(config_id: int, kind: int, index: int, step: int) -> int:
    """63-bit seed from (workload, tensor kind, matrix/group index, step)."""
    h = 0
    for v in (config_id, kind, index, step):
        h = _splitmix64(h ^ (v & _M64))
    return h & ((1 << 63) - 1)


TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


def normal_tensor(numel: int, std: float, dtype: str, key: int,
                  device: str | torch.device = "cpu") -> torch.Tensor:
    """N(0, std^2) values from a generator seeded with ``key`` on ``device``,
    cast (round-to-nearest-even) to the storage dtype."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(key)
    t = torch.randn(numel, generator=g, device=dev, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(TORCH_DTYPE[dtype])


@dataclasses.dataclass
class MuonInputs:
    params: torch.Tensor     # flat, param dtype
    grads: torch.Tensor      # flat, grad dtype
    momentum: torch.Tensor   # flat fp32


def make_muon_inputs(wl: Workload, device="cpu", step: int = 0,
                     pad: int = 0) -> MuonInputs:
    """Flat W, G and zero momentum for every matrix of ``wl``.  ``pad`` extra
    elements (filled with a sentinel) are appended after the last matrix so
    tests can check that nothing outside the matrices is written."""
    n = wl.muon_numel() + pad
    p = torch.empty(n, dtype=TORCH_DTYPE[wl.param_dtype], device=device)
    g = torch.empty(n, dtype=TORCH_DTYPE[wl.grad_dtype], device=device)
    for i, (off, r, c) in enumerate(wl.mats()):
        p[off:off + r * c] = normal_tensor(r * c, wl.w_std, wl.param_dtype,
                                           seed_key(wl.config_id, KIND_W, i, 0), device)
        g[off:off + r * c] = normal_tensor(r * c, wl.g_std, wl.grad_dtype,
                                           seed_key(wl.config_id, KIND_G, i, step), device)
    if pad:
        p[wl.muon_numel():] = 7.0
        g[wl.muon_numel():] = 7.0
    m = torch.zeros(n, dtype=torch.float32, device=device)
    if pad:
        m[wl.muon_numel():] = 7.0
    return MuonInputs(p, g, m)


def make_muon_grads(wl: Workload, step: int, device="cpu", out: torch.Tensor | None = None
                    ) -> torch.Tensor:
    """Fresh gradients for ``step`` (consecutive steps draw new gradients)."""
    n = wl.muon_numel()
    g = out if out is not None else torch.empty(n, dtype=TORCH_DTYPE[wl.grad_dtype],
                                                device=device)
    for i, (off, r, c) in enumerate(wl.mats()):
        g[off:off + r * c] = normal_tensor(r * c, wl.g_std, wl.grad_dtype,
                                           seed_key(wl.config_id, KIND_G, i, step), device)
    return g


@dataclasses.dataclass
class AdamInputs:
    param: torch.Tensor
    master: Optional[torch.Tensor]
    grad: torch.Tensor
    exp_avg: torch.Tensor
    exp_avg_sq: torch.Tensor


def make_adam_inputs(wl: Workload, gi: int, device="cpu", step: int = 0) -> AdamInputs:
    grp = wl.adam[gi]
    if grp.p_const is not None:
        master32 = torch.full((grp.numel,), grp.p_const, dtype=torch.float32, device=device)
    else:
        master32 = normal_tensor(grp.numel, grp.p_std, "fp32",
                                 seed_key(wl.config_id, KIND_ADAM_P, gi, 0), device)
    param = master32.to(TORCH_DTYPE[grp.param_dtype])
    master = master32 if grp.master else None
    if not grp.master:
        param = master32.clone()
    grad = normal_tensor(grp.numel, grp.g_std, grp.grad_dtype,
                         seed_key(wl.config_id, KIND_ADAM_G, gi, step), device)
    z = lambda: torch.zeros(grp.numel, dtype=torch.float32, device=device)  # noqa: E731
    return AdamInputs(param, master, grad, z(), z())


def make_adam_grad(wl: Workload, gi: int, step: int, device="cpu") -> torch.Tensor:
    grp = wl.adam[gi]
    return normal_tensor(grp.numel, grp.g_std, grp.grad_dtype,
                         seed_key(wl.config_id, KIND_ADAM_G, gi, step), device)


# --------------------------------------------------------------------------
# accounting (algorithmic work; no optimizer arithmetic)
# --------------------------------------------------------------------------

DTYPE_BYTES = {"bf16": 2, "fp16": 2, "fp32": 4, "int8": 1}


def ns_flops_matrix(rows: int, cols: int, steps: int, c: float) -> int:
    """Algorithmic NS flops on one matrix: per step m(m+1)n (one triangle of
    X X^T), m^2(m+1) (one triangle of A A, only when c != 0) and 2 m^2 n
    (B X), with m = min(rows, cols), n = max(rows, cols)."""
    m, n = min(rows, cols), max(rows, cols)
    per = m * (m + 1) * n + 2 * m * m * n + (m * m * (m + 1) if c != 0.0 else 0)
    return per * steps


def ns_flops_workload(wl: Workload, steps: int, c: float) -> int:
    return sum(ns_flops_matrix(r, cc, steps, c) for r, cc in wl.shapes)


def momentum_bytes_per_param(grad_dtype: str) -> int:
    """Read G and M, write M and U (in the NS operand dtype, bf16)."""
    return DTYPE_BYTES[grad_dtype] + 4 + 4 + 2


def apply_bytes_per_param(param_dtype: str, ns_dtype: str = "bf16") -> int:
    """Read W and O, write W."""
    return 2 * DTYPE_BYTES[param_dtype] + DTYPE_BYTES[ns_dtype]


def adamw_bytes_per_param(param_dtype: str, grad_dtype: str, master: bool,
                          m_dtype: str = "fp32", v_dtype: str = "fp32") -> int:
    """Read g, theta (master or param), m, v; write theta, m, v (+ param)."""
    theta = 4 if master else DTYPE_BYTES[param_dtype]
    b = DTYPE_BYTES[grad_dtype] + 2 * (theta + DTYPE_BYTES[m_dtype] + DTYPE_BYTES[v_dtype])
    if master:
        b += DTYPE_BYTES[param_dtype]
    return b


def optimizer_state_bytes(n_params: int, optimizer: str) -> int:
    """Extra optimizer-state bytes per the optimizer tutorial's memory table
    (section 2.4): SGD none, SGD-momentum one fp32 buffer, RMSProp one fp32
    buffer, Adam/AdamW two fp32 buffers, 8-bit AdamW two 8-bit buffers,
    Muon one fp32 buffer (section 4.3)."""
    per = {"sgd": 0, "sgd_momentum": 4, "rmsprop": 4, "adam": 8, "adamw": 8,
           "adamw_8bit": 2, "muon": 4}[optimizer]
    return n_params * per


if __name__ == "__main__":
    import sys
    if sys.argv[1:] == ["--freeze-ragged"]:
        write_frozen_ragged_shapes()
        print(f"wrote {RAGGED_500_JSON}")
    else:
        print("usage: python -m muon_newton_schulz_amd.workloads --freeze-ragged")
