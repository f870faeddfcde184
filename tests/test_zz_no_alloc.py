"""muon_step_noalloc (the library's static device workspace) against
muon_step with a workspace of its own: bitwise equal results on two calls
in a row, the second with a smaller input, and a plan whose workspace does
not fit is refused before anything runs."""

import pytest
import torch

import muon_newton_schulz_amd as M
from muon_newton_schulz_amd import workloads as W

pytestmark = pytest.mark.gpu

CAP = M.MUON_NOALLOC_WORKSPACE_BYTES


def _flat(shapes, gap=3):
    mats, o = [], gap
    for r, c in shapes:
        mats.append((o, r, c))
        o += r * c + gap
    return mats, o + gap


def _inputs(mats, n, dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    p = torch.full((n,), 7.0, dtype=torch.bfloat16, device=dev)
    gr = torch.full((n,), 7.0, dtype=torch.bfloat16, device=dev)
    m = torch.full((n,), 7.0, device=dev)
    for o, r, c in mats:
        p[o:o + r * c] = (torch.randn(r * c, generator=g, device=dev) * 0.02).to(torch.bfloat16)
        gr[o:o + r * c] = (torch.randn(r * c, generator=g, device=dev) * 0.02).to(torch.bfloat16)
        m[o:o + r * c] = torch.randn(r * c, generator=g, device=dev) * 1e-3
    return p, gr, m


def _hp():
    hp = W.MuonHParams()
    hp.ns_a, hp.ns_b, hp.ns_c = W.QUINTIC
    return hp


@pytest.mark.parametrize("with_out", [False, True])
def test_noalloc_step_equals_muon_step_twice(gpu, with_out):
    # the first input spans several waves under the static workspace (two
    # large matrices), with tall, off-grid and small matrices; the second,
    # smaller input then runs on the array the first left behind
    cases = [(_flat([(2048, 5632), (5632, 2048), (2048, 5632), (5632, 2048), (2048, 5632),
                     (1000, 700), (700, 1001), (96, 200)]), 31, 2),
             (_flat([(300, 520), (64, 256)]), 32, 1)]
    hp = _hp()
    for (mats, n), seed, waves in cases:
        plan = M.muon_plan_create(mats, n, "bf16", "bf16", "bf16", CAP)
        assert plan.workspace_bytes <= CAP and plan.info().n_waves == waves
        ref = _inputs(mats, n, gpu, seed)
        tst = tuple(t.clone() for t in ref)
        out_r = torch.full((n,), 7.0, device=gpu) if with_out else None
        out_t = torch.full((n,), 7.0, device=gpu) if with_out else None
        ws = plan.alloc_workspace(gpu)
        M.muon_step(plan, *ref, ws, hp, out_r)
        M.muon_step_noalloc(plan, *tst, hp, out_t)
        torch.cuda.synchronize()
        for a, b in zip(ref, tst):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
        if with_out:
            assert torch.equal(out_r, out_t)
        del ws


def test_noalloc_refuses_a_plan_too_large(gpu):
    mats, n = _flat([(8192, 8192)])   # 4 * 8192^2 bf16 workspace elements: 512 MiB
    plan = M.muon_plan_create(mats, n, "bf16", "bf16", "bf16")
    assert plan.workspace_bytes > CAP
    p, g, m = _inputs(mats, n, gpu, 33)
    p0, m0 = p.clone(), m.clone()
    with pytest.raises(M.MuonError) as e:
        M.muon_step_noalloc(plan, p, g, m, _hp())
    assert e.value.status == M.MUON_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.equal(p.view(torch.int16), p0.view(torch.int16)) and torch.equal(m, m0)
