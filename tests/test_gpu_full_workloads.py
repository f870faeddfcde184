"""GPU parity on the two largest workloads at their full size, in the launch
configuration the benchmark times: one plan over every matrix, one wave, the
update fused into the last NS phase.

* ``moe_e384_7168x2048``: 1152 expert matrices (gate, up 7168x2048; down
  2048x7168) in one flat buffer of 1.69e10 elements (MoonEP news item,
  memory contract: [E, H, H'] blocks addressed by offset).
* ``ragged_500``: 500 ragged matrices (1.01e10 elements, every tenth off the
  64 grid, so most offsets are odd) plus AdamW on a 163840 x 7168 embedding
  and 128 vectors (the K2 answer's flat concatenation, section 2.2).

Both flat buffers reach past 2^31 and 2^32 elements, and their workspaces
(87 and 75 GB) put the later matrices' NS operands past 2^32 elements.  The
oracle checks sampled matrices whole: the first and last of each buffer,
the ones that straddle element 2^31 and 2^32, the largest, off-grid tall and
wide matrices, and matrices whose rows lie on the flat buffer's 8-element
grid and off it (the fused update writes the latter realigned).  The first
ragged step writes O out, so the apply kernel updates every matrix there.

Checks per sampled matrix (tolerances as in test_gpu_parity.py):
  M (fp32) <= 2e-6; O <= 1e-2 where O is written out (out_update);
  X after 4 iterations (exported from the workspace) <= 1e-2;
  W (bf16) through the update it implies: with the fused update the step
  writes W1 = RNE(decay W0 - step O) and no O, so O_impl = (decay W0 - W1) /
  step differs from the GPU's O by at most half a bf16 ulp of W1 per
  element over step; the check is ||O_impl - O_ref|| <= 1e-2 ||O_ref|| +
  ||ulp(W1) / 2|| / step (triangle inequality).
"""

import math

import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as M
from muon_newton_schulz_amd import workloads as W
from oracle import muon_oracle as O

pytestmark = pytest.mark.gpu

TOL_O = 1e-2


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def ohp(hp):
    return O.MuonHP(lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                    nesterov=hp.nesterov, ns_a=hp.ns_a, ns_b=hp.ns_b, ns_c=hp.ns_c,
                    ns_steps=hp.ns_steps, eps=hp.eps, scale_mode=hp.scale_mode,
                    rms_target=hp.rms_target)


def quintic_hp():
    hp = W.MuonHParams()
    hp.ns_a, hp.ns_b, hp.ns_c = W.QUINTIC
    return hp


def half_ulp_bf16(x):
    """Half a bf16 ulp of each (bf16-representable) value: 2^(e - 8) for
    |x| in [2^e, 2^(e+1)); the smallest normal's for zeros."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8)


def straddling(mats, x):
    return next(i for i, (o, r, c) in enumerate(mats) if o < x <= o + r * c - 1)


class Sample:
    """Host copies of one matrix's state before a step."""

    def __init__(self, inp, mat):
        o, r, c = mat
        sl = slice(o, o + r * c)
        self.r, self.c, self.sl = r, c, sl
        self.W0 = np64(inp.params[sl]).reshape(r, c)
        self.G = np64(inp.grads[sl]).reshape(r, c)
        self.M0 = np64(inp.momentum[sl]).reshape(r, c)


def check_sample(tag, s, inp, hp, out=None):
    """Oracle step from the sample's state; checks M, W (through the implied
    update) and, when given, the written-out O.  Returns the oracle's X0."""
    print(f"oracle {tag} {s.r}x{s.c}", flush=True)
    ref_W, ref_M, ref_O = O.muon_matrix_math(s.W0, s.G, s.M0, ohp(hp))
    M1 = np64(inp.momentum[s.sl]).reshape(s.r, s.c)
    W1 = np64(inp.params[s.sl]).reshape(s.r, s.c)
    assert rel(M1, O.fp32_round(ref_M)) <= 2e-6, (tag, "M")
    if out is not None:
        assert rel(np64(out[s.sl]).reshape(s.r, s.c), ref_O) <= TOL_O, (tag, "O")
    # the GPU's decay and step, in its fp32 arithmetic
    decay = float(np.float32(1.0) - np.float32(hp.lr) * np.float32(hp.weight_decay))
    scale = hp.rms_target * math.sqrt(max(s.r, s.c))
    step = float(np.float32(hp.lr) * np.float32(scale))
    O_impl = (decay * s.W0 - W1) / step
    slack = np.linalg.norm(half_ulp_bf16(W1)) / (step * np.linalg.norm(ref_O))
    e = rel(O_impl, ref_O)
    assert e <= TOL_O + slack, (tag, "W", e, slack)
    U = O.nesterov_lookahead(ref_M, s.G, hp.momentum, hp.nesterov)
    return O.frobenius_normalise(U, hp.eps)


def check_x4(tag, s, x0, xout, hp):
    """X after 4 NS iterations, exported from the workspace."""
    print(f"oracle {tag} X4 {s.r}x{s.c}", flush=True)
    ref = O.newton_schulz(x0, hp.ns_a, hp.ns_b, hp.ns_c, 4)
    assert rel(np64(xout[s.sl]).reshape(s.r, s.c), ref) <= TOL_O, (tag, "X4")


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_moe_e384_full_workload(gpu):
    wl = W.workload("moe_e384_7168x2048")
    mats = wl.mats()
    assert len(mats) == 1152 and mats[-1][0] > 2 ** 33
    i31, i32 = straddling(mats, 2 ** 31), straddling(mats, 2 ** 32)
    # first and last of each projection block (gate and up tall, down wide),
    # the matrices across elements 2^31 and 2^32
    sample = sorted({0, i31, i32, 767, 768, 1151})
    hp = quintic_hp()
    inp = W.make_muon_inputs(wl, gpu, step=1)
    plan = M.muon_plan_create(mats, wl.muon_numel(), "bf16", "bf16", "bf16")
    info = plan.info()
    assert info.n_waves == 1 and info.fused_apply_mats == 1152
    ws = plan.alloc_workspace(gpu)
    assert plan.workspace_bytes > 2 * 2 ** 33   # later operands past 2^32 bf16 elements
    before = {i: Sample(inp, mats[i]) for i in sample}
    M.muon_step(plan, inp.params, inp.grads, inp.momentum, ws, hp)   # fused update
    torch.cuda.synchronize()
    x0 = {i: check_sample(("e384", i), before[i], inp, hp) for i in sample}
    # X after 4 iterations is still in the workspace (the fused last phase
    # wrote W instead of X'): export it over the gradient buffer's memory
    inp.grads = None
    _free()
    xout = torch.zeros(wl.muon_numel(), dtype=torch.float32, device=gpu)
    M.muon_stage_export_x(plan, 0, ws, 4, xout)
    torch.cuda.synchronize()
    for i in sample:
        check_x4(("e384", i), before[i], x0[i], xout, hp)
    del xout, ws, inp, plan
    _free()


@pytest.mark.timeout(900)
def test_ragged_500_full_mixed_workload(gpu):
    wl = W.workload("ragged_500")
    mats = wl.mats()
    i31 = straddling(mats, 2 ** 31)
    flops = [W.ns_flops_matrix(r, c, 5, 1.0) for _, r, c in mats]
    largest = max(range(len(mats)), key=lambda i: flops[i])
    offgrid = [i for i, (o, r, c) in enumerate(mats) if (r % 64 or c % 64) and o > 2 ** 32]
    tall_off = min((i for i in offgrid if mats[i][1] > mats[i][2]), key=lambda i: flops[i])
    wide_off = min((i for i in offgrid if mats[i][1] < mats[i][2]), key=lambda i: flops[i])
    ongrid = [i for i, (o, r, c) in enumerate(mats) if o % 8 == 0 and c % 8 == 0 and o > 2 ** 32]
    ongrid_small = sorted(ongrid, key=lambda i: flops[i])[:2]
    step1 = sorted({0, i31, largest, tall_off, wide_off, *ongrid_small, len(mats) - 1})
    step2 = sorted({i31, tall_off, wide_off, *ongrid_small})
    hp = quintic_hp()

    inp = W.make_muon_inputs(wl, gpu, step=1)
    adam = [W.make_adam_inputs(wl, gi, device=gpu, step=1) for gi in range(len(wl.adam))]
    plan = M.muon_plan_create(mats, wl.muon_numel(), "bf16", "bf16", "bf16")
    info = plan.info()
    assert info.n_waves == 1 and info.fused_apply_mats == len(mats) - info.small_mats
    ws = plan.alloc_workspace(gpu)
    out = torch.zeros(wl.muon_numel(), dtype=torch.float32, device=gpu)

    # AdamW samples: start, middle and end of each group
    def adam_slices(n):
        return [slice(0, min(n, 4096)), slice(n // 2 - 2049, n // 2 + 2049),
                slice(max(0, n - 4097), n)]

    a_state = []
    for a, grp in zip(adam, wl.adam):
        sls = adam_slices(grp.numel)
        a_state.append([(np64(a.param[s]), np64(a.master[s]), np.zeros(s.stop - s.start),
                         np.zeros(s.stop - s.start)) for s in sls])
    ahp = O.AdamWHP(wl.adam_hp.lr, wl.adam_hp.beta1, wl.adam_hp.beta2, wl.adam_hp.eps,
                    wl.adam_hp.weight_decay)

    def adam_step_and_check(t):
        for gi, (a, grp) in enumerate(zip(adam, wl.adam)):
            g = W.make_adam_grad(wl, gi, t, device=gpu)
            M.adamw_step(a.param, a.master, g, a.exp_avg, a.exp_avg_sq, wl.adam_hp, t)
            torch.cuda.synchronize()
            for k, s in enumerate(adam_slices(grp.numel)):
                p0, m0, e0, v0 = a_state[gi][k]
                pr, mr, er, vr = O.adamw_step_stored(p0, m0, np64(g[s]), e0, v0, ahp, t, "bf16")
                master = np64(a.master[s])
                assert rel(master, mr) <= 2e-6, (grp.name, t, k)
                assert rel(np64(a.exp_avg[s]), er) <= 2e-6, (grp.name, t, k)
                assert rel(np64(a.exp_avg_sq[s]), vr) <= 2e-6, (grp.name, t, k)
                np.testing.assert_array_equal(np64(a.param[s]), O.bf16_round(master))
                a_state[gi][k] = (np64(a.param[s]), master, np64(a.exp_avg[s]),
                                  np64(a.exp_avg_sq[s]))
            del g

    # step 1: O written out (the separate apply kernel for every matrix)
    before = {i: Sample(inp, mats[i]) for i in step1}
    M.muon_step(plan, inp.params, inp.grads, inp.momentum, ws, hp, out)
    torch.cuda.synchronize()
    for i in step1:
        check_sample(("ragged step 1", i), before[i], inp, hp, out)
    adam_step_and_check(1)

    # step 2 from the new state, fresh gradients, as timed: the update fused
    # into the last NS phase (realigned for the off-grid matrices)
    W.make_muon_grads(wl, 2, gpu, out=inp.grads)
    before = {i: Sample(inp, mats[i]) for i in step2}
    M.muon_step(plan, inp.params, inp.grads, inp.momentum, ws, hp)
    torch.cuda.synchronize()
    x0 = {i: check_sample(("ragged step 2", i), before[i], inp, hp) for i in step2}
    M.muon_stage_export_x(plan, 0, ws, 4, out)
    torch.cuda.synchronize()
    for i in step2:
        check_x4(("ragged step 2", i), before[i], x0[i], out, hp)
    adam_step_and_check(2)
    del out, ws, inp, adam, plan
    _free()
