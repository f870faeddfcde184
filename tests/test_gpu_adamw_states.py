"""GPU parity of AdamW with compressed optimizer states (adamw_step_ex: m in
fp32 or bf16, v in fp32, bf16 or fp16) against the fp64 oracle with the
same storage types (reading R13).

Tolerances, per step, each step started from the GPU's own stored state
(the oracle is fed the GPU's m, v and master from before the step):
  every stored state is within one storage ulp of the oracle's, plus 1e-6
    of the magnitude of the two terms of its update (the fp32 kernel's
    pre-rounding error; where the terms cancel it is the larger part), and
    at most 3% of the 16-bit states differ at all.
    Why they can differ at all: with m and g both bf16, b1 m + (1 - b1) g is
    often exactly halfway between two bf16 values in real arithmetic, and
    the fp64 oracle (beta1 = 0.9 as fp64) and the fp32 kernel (beta1 = 0.9
    as fp32, 1 - beta1 computed in fp32) land on opposite sides of the tie.
    An fp32 emulation of the kernel puts such flips at <= 1.6% of the
    elements per step for m and <= 0.8% for v on these inputs.
  master and params: 2e-6 relative (the hyper-parameters reach the kernel
    as fp32: 1 - beta2 alone differs from the fp64 value by 2.4e-7
    relative).
"""

import ctypes

import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as M
from muon_newton_schulz_amd import workloads as W
from oracle import muon_oracle as O

from test_gpu_parity import np64, rel

pytestmark = pytest.mark.gpu

TORCH = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def _randn(n, dtype, dev, seed, std=1.0):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn(n, generator=g, device=dev) * std).to(dtype)


def _ahp():
    hp = W.AdamWHParams()
    return hp, O.AdamWHP(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)


def _spacing(x, dt):
    """Distance from |x| to the next larger value of the storage type."""
    bits, emin = {"bf16": (8, -126), "fp16": (11, -14)}[dt]
    _, e = np.frexp(np.abs(x))          # |x| in [2^(e-1), 2^e)
    e = np.where(x == 0, emin + 1, e)   # at zero: the smallest subnormal
    return np.ldexp(1.0, np.maximum(e - 1, emin) - (bits - 1))


def _bound(got, want, dt, terms):
    """How far the stored state may sit from the oracle's: one storage ulp
    either side (each side rounds its own pre-rounding value to nearest)
    plus how far the kernel's fp32 pre-rounding value b m + (1 - b) x can
    sit from the exact one: 1e-6 of the magnitude of the two terms (beta
    and 1 - beta as fp32 differ from the fp64 values by up to 2.4e-7
    relative; three fp32 roundings add 1.8e-7).  The terms, not the
    result, set that scale: where they cancel the result's relative error
    is unbounded."""
    if dt == "fp32":
        ulp = 2.0 ** -23 * np.maximum(np.abs(got), np.abs(want))
    else:
        ulp = np.maximum(_spacing(got, dt), _spacing(want, dt))
    return ulp + 1e-6 * terms


STATE_CASES = [("bf16", "fp32"), ("fp32", "bf16"), ("fp32", "fp16"), ("bf16", "fp16"),
               ("bf16", "bf16")]


def _check_state(got, want, dt, what, terms):
    r = np.abs(got - want) / _bound(got, want, dt, terms)
    if not np.all(r <= 1.0):
        i = int(np.argmax(r))
        pytest.fail(f"{what}: {int(np.count_nonzero(r > 1))} elements beyond the bound; worst "
                    f"#{i} got {got[i]!r} want {want[i]!r} ({r[i]:.3g} x the bound)")
    if dt != "fp32":
        assert np.count_nonzero(got != want) <= 0.03 * got.size, what


def _terms(hp, m0, v0, g, f=1.0):
    g = f * g
    return (hp.beta1 * np.abs(m0) + (1 - hp.beta1) * np.abs(g),
            hp.beta2 * np.abs(v0) + (1 - hp.beta2) * g * g)


@pytest.mark.parametrize("mdt,vdt", STATE_CASES)
@pytest.mark.parametrize("pdt", ["bf16", "fp32"])
def test_compressed_states_ten_steps(gpu, mdt, vdt, pdt):
    n = 100003
    hp, ohp = _ahp()
    master = _randn(n, torch.float32, gpu, 1, 0.02)
    params = master.to(TORCH[pdt]) if pdt == "bf16" else master.clone()
    mst = master if pdt == "bf16" else None
    m = torch.zeros(n, dtype=TORCH[mdt], device=gpu)
    v = torch.zeros(n, dtype=TORCH[vdt], device=gpu)
    for t in range(1, 11):
        g = _randn(n, torch.bfloat16, gpu, 100 + t, 0.02)
        p0, th0, m0, v0 = np64(params), np64(master), np64(m), np64(v)
        M.adamw_step(params, mst, g, m, v, hp, t)
        torch.cuda.synchronize()
        rp, rth, rm, rv = O.adamw_step_stored(p0, th0 if mst is not None else None, np64(g),
                                              m0, v0, ohp, t, pdt, m_dtype=mdt, v_dtype=vdt)
        tm, tv = _terms(ohp, m0, v0, np64(g))
        _check_state(np64(m), rm, mdt, f"m step {t}", tm)
        _check_state(np64(v), rv, vdt, f"v step {t}", tv)
        if mst is not None:
            assert rel(np64(master), rth) <= 2e-6, t
            # the bf16 parameter is the cast of the stored master
            assert np.array_equal(np64(params), O.bf16_round(np64(master)))
        else:
            assert rel(np64(params), rp) <= 2e-6, t


def test_fp16_second_moment_underflow_matches_oracle(gpu):
    # gradients of 1e-4: (1 - b2) g^2 ~ 5e-10 is below fp16's smallest
    # subnormal; the stored v underflows to 0 on both sides
    n = 4096 + 5
    hp, ohp = _ahp()
    p = _randn(n, torch.float32, gpu, 7)
    m = torch.zeros(n, device=gpu)
    v = torch.zeros(n, dtype=torch.float16, device=gpu)
    g = _randn(n, torch.float32, gpu, 8, 1e-4)
    p0 = np64(p)
    M.adamw_step(p, None, g, m, v, hp, 1)
    torch.cuda.synchronize()
    rp, _, rm, rv = O.adamw_step_stored(p0, None, np64(g), np.zeros(n), np.zeros(n), ohp, 1,
                                        "fp32", v_dtype="fp16")
    assert np.count_nonzero(rv) < n // 100  # the oracle underflows too
    assert np.array_equal(np64(v) == 0, rv == 0)
    _check_state(np64(v), rv, "fp16", "v", _terms(ohp, 0.0, 0.0, np64(g))[1])
    assert rel(np64(p), rp) <= 2e-6


def test_adamw_step_is_adamw_step_ex_with_fp32_states(gpu):
    n = 10007
    hp, _ = _ahp()
    a_p, b_p = _randn(n, torch.float32, gpu, 9), _randn(n, torch.float32, gpu, 9)
    g = _randn(n, torch.bfloat16, gpu, 10)
    a_m, a_v, b_m, b_v = (torch.zeros(n, device=gpu) for _ in range(4))
    h = M._ahp(hp)
    L = M.lib()
    stream = torch.cuda.current_stream().cuda_stream
    assert L.adamw_step(a_p.data_ptr(), 0, None, g.data_ptr(), 1, a_m.data_ptr(), a_v.data_ptr(),
                        n, ctypes.byref(h), 1, stream) == 0
    assert L.adamw_step_ex(b_p.data_ptr(), 0, None, g.data_ptr(), 1, b_m.data_ptr(), 0,
                           b_v.data_ptr(), 0, n, ctypes.byref(h), 1, stream) == 0
    torch.cuda.synchronize()
    for x, y in ((a_p, b_p), (a_m, b_m), (a_v, b_v)):
        assert torch.equal(x, y)


def test_unaligned_compressed_states_and_clip(gpu):
    # offsets by one element: the scalar path; with a clip scale
    n = 5001
    hp, ohp = _ahp()
    pb = _randn(n + 1, torch.float32, gpu, 11)
    mb = torch.zeros(n + 1, dtype=torch.bfloat16, device=gpu)
    vb = torch.zeros(n + 1, dtype=torch.float16, device=gpu)
    g = _randn(n + 1, torch.bfloat16, gpu, 12, 0.5)[1:]
    p, m, v = pb[1:], mb[1:], vb[1:]
    clip = M.grad_norm_clip([g], 1.0)
    f = M.read_clip_state(clip)["scale"]
    assert f < 1.0
    p0 = np64(p)
    M.adamw_step(p, None, g, m, v, hp, 1, clip=clip)
    torch.cuda.synchronize()
    rp, _, rm, rv = O.adamw_step_stored(p0, None, np64(g), np.zeros(n), np.zeros(n), ohp, 1,
                                        "fp32", grad_scale=f, m_dtype="bf16", v_dtype="fp16")
    tm, tv = _terms(ohp, 0.0, 0.0, np64(g), f)
    _check_state(np64(m), rm, "bf16", "m", tm)
    _check_state(np64(v), rv, "fp16", "v", tv)
    assert rel(np64(p), rp) <= 2e-6
    assert np64(pb)[0] == np64(_randn(n + 1, torch.float32, gpu, 11))[0]  # untouched
