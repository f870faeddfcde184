"""GPU parity of gradient clipping, the non-finite step guard and the
optimizer-state statistics (through the C ABI) against the fp64 oracle in
oracle/guard_oracle.py.

Tolerances:
  global norm (stored in fp32)        relative 1e-6 (one fp32 rounding)
  clip scale (stored in fp32)         relative 1e-6
  skip flag, counts                   exact
  statistics mean / var               relative 1e-9 (fp64, different order)
  statistics min / max / max |x|      exact (order-free)
  clipped Muon and AdamW steps        the step tolerances of test_gpu_parity
  guarded (skipped) steps, scale 1    bitwise: nothing changes / equal to
                                      the unclipped step
"""

import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as M
from muon_newton_schulz_amd import workloads as W
from oracle import guard_oracle as G
from oracle import muon_oracle as O

from test_gpu_parity import QUINTIC, Setup, check_muon_step, mhp, np64, ohp, rel

pytestmark = pytest.mark.gpu


def _randn(n, dtype, dev, seed, std=1.0):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn(n, generator=g, device=dev) * std).to(dtype)


def _buffers(dev):
    """Gradient buffers of both dtypes, aligned and not, with ragged tails."""
    big = _randn(1 << 22, torch.bfloat16, dev, 1, 0.02)
    odd = _randn(1000003 + 1, torch.bfloat16, dev, 2, 0.5)[1:]        # 2-byte aligned only
    f32 = _randn(4096 * 37 + 5, torch.float32, dev, 3, 1e-3)
    f32u = _randn(777 + 1, torch.float32, dev, 4, 3.0)[1:]           # 4-byte aligned only
    empty = torch.zeros(0, dtype=torch.bfloat16, device=dev)
    return [big, odd, f32, empty, f32u]


def test_grad_norm_and_scale_match_oracle(gpu):
    bufs = _buffers(gpu)
    ref = G.global_grad_norm([np64(b) for b in bufs])
    for max_norm in (0.5 * ref, 2.0 * ref, 0.0):
        out = M.grad_norm_clip(bufs, max_norm)
        st = M.read_clip_state(out)
        assert not st["skip"]
        assert abs(st["norm"] - ref) <= 1e-6 * ref, (st["norm"], ref)
        want = G.clip_factor(ref, max_norm)
        assert abs(st["scale"] - want) <= 1e-6 * want, (max_norm, st["scale"], want)
    # bitwise reproducible
    a = M.grad_norm_clip(bufs, 1.0).cpu()
    b = M.grad_norm_clip(bufs, 1.0).cpu()
    assert torch.equal(a, b)
    # no buffers: norm 0, scale 1
    st = M.read_clip_state(M.grad_norm_clip([], 1.0))
    assert st == {"norm": 0.0, "scale": 1.0, "skip": False}


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), float("-inf")])
def test_guard_trips_on_non_finite(gpu, bad):
    bufs = _buffers(gpu)
    bufs[2][12345] = bad
    st = M.read_clip_state(M.grad_norm_clip(bufs, 1.0))
    assert st["skip"] and st["scale"] == 1.0
    assert G.guard_skip(G.global_grad_norm([np64(b) for b in bufs]))


def _muon_setup(gpu, pdt, ns_dtype, seed):
    shapes = [(96, 200), (200, 96), (129, 257), (64, 64), (17, 300)]
    mats, o = [], 5
    for r, c in shapes:
        mats.append((o, r, c))
        o += r * c + 5
    return Setup(mats, o, pdt, pdt, ns_dtype, gpu, seed=seed)


@pytest.mark.parametrize("ns_dtype,pdt", [("bf16", "bf16"), ("fp32", "fp32")])
def test_clipped_muon_step_matches_oracle(gpu, ns_dtype, pdt):
    s = _muon_setup(gpu, pdt, ns_dtype, 11)
    hp = mhp(QUINTIC)
    g_sel = torch.cat([s.grads[o:o + r * c] for (o, r, c) in s.mats])
    ref = G.global_grad_norm([np64(g_sel)])
    max_norm = 0.25 * ref
    clip = M.grad_norm_clip([s.grads[o:o + r * c] for (o, r, c) in s.mats], max_norm)
    f = G.clip_factor(ref, max_norm)
    assert f < 0.3
    P0, G0, M0 = s.snapshot()
    M.muon_step(s.plan, s.params, s.grads, s.mom, s.ws, hp, s.out, clip=clip)
    torch.cuda.synchronize()
    Pr, Mr, outs = O.muon_step_flat(P0, G0, M0, s.mats, ohp(hp), pdt, grad_scale=f)
    P1, M1, Og = np64(s.params), np64(s.mom), np64(s.out)
    for i, (o, r, c) in enumerate(s.mats):
        sl = slice(o, o + r * c)
        assert rel(M1[sl], Mr[sl]) <= 2e-6, (i, "M")
        assert rel(Og[sl].reshape(r, c), outs[i]) <= (1e-2 if ns_dtype == "bf16" else 1e-4)
        assert rel(P1[sl], Pr[sl]) <= (1e-2 if pdt == "bf16" else 1e-4), (i, "W")


def test_clipped_adamw_matches_oracle(gpu):
    n = 50000 + 3
    p = _randn(n, torch.float32, gpu, 21)
    g = _randn(n, torch.float32, gpu, 22, 0.1)
    m = torch.zeros(n, device=gpu)
    v = torch.zeros(n, device=gpu)
    hp = W.AdamWHParams()
    ref = G.global_grad_norm([np64(g)])
    clip = M.grad_norm_clip([g], 0.1 * ref)
    f = G.clip_factor(ref, 0.1 * ref)
    p0, g0 = np64(p), np64(g)
    for t in (1, 2, 3):
        M.adamw_step(p, None, g, m, v, hp, t, clip=clip)
    torch.cuda.synchronize()
    th, mm, vv = p0, np.zeros(n), np.zeros(n)
    ahp = O.AdamWHP(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
    for t in (1, 2, 3):
        th, _, mm, vv = O.adamw_step_stored(th, None, g0, mm, vv, ahp, t, "fp32", grad_scale=f)
    assert rel(np64(p), th) <= 2e-6
    assert rel(np64(m), mm) <= 2e-6
    assert rel(np64(v), vv) <= 2e-6


def test_skipped_step_changes_nothing(gpu):
    s = _muon_setup(gpu, "bf16", "bf16", 31)
    o0, r0, c0 = s.mats[2]
    s.grads[o0 + 77] = float("nan")
    n = 4099
    ap = _randn(n, torch.bfloat16, gpu, 32)
    am = _randn(n, torch.float32, gpu, 33)
    ag = _randn(n, torch.bfloat16, gpu, 34)
    ag[5] = float("inf")
    m1 = _randn(n, torch.float32, gpu, 35)
    v1 = _randn(n, torch.float32, gpu, 36).abs()
    clip = M.grad_norm_clip([s.grads, ag], 1.0)
    before = [t.clone() for t in (s.params, s.mom, s.out, ap, am, m1, v1)]
    M.muon_step(s.plan, s.params, s.grads, s.mom, s.ws, mhp(QUINTIC), s.out, clip=clip)
    M.adamw_step(ap, am, ag, m1, v1, W.AdamWHParams(), 1, clip=clip)
    torch.cuda.synchronize()
    assert M.read_clip_state(clip)["skip"]
    for b, a in zip(before, (s.params, s.mom, s.out, ap, am, m1, v1)):
        assert torch.equal(b, a)


def test_scale_one_is_bitwise_the_unclipped_step(gpu):
    a = _muon_setup(gpu, "bf16", "bf16", 41)
    b = _muon_setup(gpu, "bf16", "bf16", 41)
    clip = M.grad_norm_clip([a.grads], 1e30)
    assert M.read_clip_state(clip)["scale"] == 1.0
    hp = mhp(QUINTIC)
    M.muon_step(a.plan, a.params, a.grads, a.mom, a.ws, hp, a.out, clip=clip)
    M.muon_step(b.plan, b.params, b.grads, b.mom, b.ws, hp, b.out)
    n = 3001
    p1, p2 = _randn(n, torch.float32, gpu, 42), _randn(n, torch.float32, gpu, 42)
    g = _randn(n, torch.bfloat16, gpu, 43)
    m1, m2, v1, v2 = (torch.zeros(n, device=gpu) for _ in range(4))
    M.adamw_step(p1, None, g.float(), m1, v1, W.AdamWHParams(), 1, clip=clip)
    M.adamw_step(p2, None, g.float(), m2, v2, W.AdamWHParams(), 1)
    torch.cuda.synchronize()
    for x, y in ((a.params, b.params), (a.mom, b.mom), (a.out, b.out), (p1, p2), (m1, m2),
                 (v1, v2)):
        assert torch.equal(x, y)


def _check_stats(x, ref):
    st = M.read_state_stats(M.state_stats(x))
    assert st["count"] == ref["count"] and st["nonfinite"] == ref["nonfinite"]
    for k in ("min", "max", "absmax"):
        assert st[k] == ref[k], (k, st[k], ref[k])
    assert abs(st["mean"] - ref["mean"]) <= 1e-9 * max(abs(ref["mean"]), ref["absmax"] * 1e-3, 1e-300)
    assert abs(st["var"] - ref["var"]) <= 1e-9 * max(ref["var"], 1e-300)
    return st


def test_state_stats_match_oracle(gpu):
    x = _randn(3 * 1024 * 1024 + 7, torch.float32, gpu, 51, 0.01) + 0.003
    x[17] = float("nan")
    x[1 << 20] = float("inf")
    x[-1] = float("-inf")
    _check_stats(x, G.state_stats(np64(x)))
    xu = x[1:1000001]  # 4-byte aligned only
    _check_stats(xu, G.state_stats(np64(xu)))
    # second-moment-like: positive, spread over orders of magnitude
    v = torch.exp(_randn(777777, torch.float32, gpu, 52, 4.0))
    _check_stats(v, G.state_stats(np64(v)))
    # bitwise reproducible
    assert torch.equal(M.state_stats(x).cpu(), M.state_stats(x).cpu())


def test_state_stats_edge_cases(gpu):
    empty = torch.zeros(0, device=gpu)
    st = M.read_state_stats(M.state_stats(empty))
    assert st["count"] == 0 and st["nonfinite"] == 0 and st["mean"] == 0.0 and st["var"] == 0.0
    nan = torch.full((1000,), float("nan"), device=gpu)
    st = M.read_state_stats(M.state_stats(nan))
    assert st["count"] == 0 and st["nonfinite"] == 1000 and st["min"] == 0.0
    const = torch.full((123457,), -2.5, device=gpu)
    st = M.read_state_stats(M.state_stats(const))
    assert st["mean"] == -2.5 and st["var"] == 0.0 and st["absmax"] == 2.5
    one = torch.tensor([3.0], device=gpu)
    st = M.read_state_stats(M.state_stats(one))
    assert st == {"mean": 3.0, "var": 0.0, "min": 3.0, "max": 3.0, "absmax": 3.0, "count": 1,
                  "nonfinite": 0}


def test_dense_stack_gradient_norm_full_size(gpu):
    """The global norm over every gradient of the dense d2048 x 16 stack
    (Muon flat buffer + the AdamW groups), clip scale from it."""
    wl = W.workload("dense_d2048_l16")
    grads = W.make_muon_grads(wl, step=1, device=gpu)
    adam = [W.make_adam_grad(wl, k, step=1, device=gpu) for k in range(len(wl.adam))]
    bufs = [grads] + adam
    st = M.read_clip_state(M.grad_norm_clip(bufs, 1.0))
    ref = G.global_grad_norm([np64(b) for b in bufs])
    assert abs(st["norm"] - ref) <= 1e-6 * ref
    assert abs(st["scale"] - G.clip_factor(ref, 1.0)) <= 1e-6
