"""The update applied by the last NS phase (muon_stage_ns_apply, and
muon_step without out_update) against the separate apply kernel (muon_step
with out_update, muon_stage_apply): params and momentum must be bitwise
equal.  Both compute W' = fma(-step, O, decay * W) from the same bf16 O, so
the fused path needs no tolerance of its own; the unfused path is checked
against the oracle in test_gpu_parity.py.

Every tiled matrix is fused when the NS and the params are bf16 and the
parameter buffer is 16-byte aligned.  Wide matrices write W rows from the
tile rows, tall ones through a transposed pass.  When a matrix's offset or
cols are off the 8-element grid, its W rows are realigned: 16-byte pieces
on the grid, the parameters before and after them one by one.  The small
matrices keep the apply kernel.
"""

import pytest
import torch

import muon_newton_schulz_amd as M
from muon_newton_schulz_amd import workloads as W

from test_gpu_parity import CUBIC, QUINTIC, mhp

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16

# (rows, cols, tiled): every tiled matrix takes the fused update
SHAPES = [
    (256, 512, True),     # wide, on the grid
    (520, 296, True),     # tall (transposed pass), cols % 8 == 0
    (520, 300, True),     # tall, cols % 8 == 4: realigned rows
    (700, 1000, True),    # wide, rows off the tile grid
    (1000, 776, True),    # tall, rows off the grid
    (1000, 700, True),    # tall, cols % 8 == 4
    (129, 8, False),      # small-matrix path
    (64, 64, False),      # small-matrix path
    (2048, 5632, True),
    (5632, 2048, True),
    (300, 520, True),     # offset made odd below: realigned rows
    (330, 1024, True),    # wide, last tile row half padding (half-height tiles)
    (256, 1096, True),    # wide, last tile column half padding (half-width tiles)
]


def _layout(shapes, misalign=(10,)):
    mats, o, fused = [], 16, 0
    for k, (r, c, f) in enumerate(shapes):
        if k in misalign:
            o += 3                         # an offset that is not a multiple of 8
        mats.append((o, r, c))
        fused += int(f)
        o += r * c
        o = (o + 7) // 8 * 8 + 8           # next offset aligned (gaps stay untouched)
    return mats, o + 8, fused


class Case:
    def __init__(self, gpu, mats, n, seed, pdt="bf16"):
        g = torch.Generator(device=gpu)
        g.manual_seed(seed)
        dt = W.TORCH_DTYPE[pdt]
        self.params = (torch.randn(n, generator=g, device=gpu) * 0.02).to(dt)
        self.grads = (torch.randn(n, generator=g, device=gpu) * 0.02).to(BF16)
        self.mom = torch.zeros(n, device=gpu)
        self.plan = M.muon_plan_create(mats, n, pdt, "bf16", "bf16")
        self.ws = self.plan.alloc_workspace(gpu)
        self.out = torch.zeros(n, device=gpu)


@pytest.mark.parametrize("coef", [QUINTIC, CUBIC])
def test_fused_step_is_bitwise_the_apply_kernel(gpu, coef):
    mats, n, n_fused = _layout(SHAPES)
    a = Case(gpu, mats, n, 5)
    b = Case(gpu, mats, n, 5)
    assert a.plan.info().fused_apply_mats == n_fused == 11
    hp = mhp(coef)
    p0 = a.params.clone()
    for _ in range(2):  # the second step starts from a nonzero momentum
        M.muon_step(a.plan, a.params, a.grads, a.mom, a.ws, hp)            # fused
        M.muon_step(b.plan, b.params, b.grads, b.mom, b.ws, hp, b.out)     # apply kernel
    torch.cuda.synchronize()
    assert torch.equal(a.params.view(torch.int16), b.params.view(torch.int16))
    assert torch.equal(a.mom, b.mom)
    assert not torch.equal(a.params, p0)


# every offset off the 8-element grid (odd shifts 1, 3, 5, 7 in turn), so
# each W row starts at a different position within a 16-byte piece
OFFGRID = [
    (330, 1100),    # wide: half-height and half-width edge tiles
    (1100, 330),    # tall: the same, through the transposed pass
    (333, 1031),    # wide, odd cols
    (1031, 333),    # tall, odd cols
    (257, 2307),    # wide, one row into a second tile row
    (2307, 257),    # tall
    (3, 40000),     # wide, 3 rows (tiled: 40000 columns)
    (40000, 3),     # tall, 3 columns: every W row shorter than a piece
    (1500, 1501),   # square-ish, several tiles per side
]


def _offgrid_layout():
    mats, o = [], 16
    for k, (r, c) in enumerate(OFFGRID):
        o += 2 * (k % 4) + 1
        mats.append((o, r, c))
        o += r * c
    return mats, o   # the last matrix ends the buffer


@pytest.mark.parametrize("coef", [QUINTIC, CUBIC])
def test_offgrid_rows_fused_bitwise_the_apply_kernel(gpu, coef):
    mats, n = _offgrid_layout()
    guard = 64
    res = []
    plan = M.muon_plan_create(mats, n, "bf16", "bf16", "bf16")
    info = plan.info()
    assert info.fused_apply_mats == len(mats) and info.small_mats == 0
    ws = plan.alloc_workspace(gpu)
    for fused in (True, False):
        g = torch.Generator(device=gpu)
        g.manual_seed(31)
        # `guard` elements past the buffer, which ends with the last matrix
        base = (torch.randn(n + guard, generator=g, device=gpu) * 0.02).to(BF16)
        grads = (torch.randn(n, generator=g, device=gpu) * 0.02).to(BF16)
        mom = torch.zeros(n, device=gpu)
        out = None if fused else torch.zeros(n, device=gpu)
        p0 = base.clone()
        for _ in range(2):
            M.muon_step(plan, base[:n], grads, mom, ws, mhp(coef), out)
        torch.cuda.synchronize()
        # the gaps between matrices and the elements past the buffer are
        # untouched; every matrix changed
        covered = torch.zeros(n + guard, dtype=torch.bool, device=gpu)
        for o, r, c in mats:
            covered[o:o + r * c] = True
            assert not torch.equal(base[o:o + r * c], p0[o:o + r * c])
        assert torch.equal(base[~covered].view(torch.int16), p0[~covered].view(torch.int16))
        res.append((base.view(torch.int16).clone(), mom.clone()))
    assert torch.equal(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1])


@pytest.mark.parametrize("steps", [0, 1, 2])
def test_fused_step_few_iterations(gpu, steps):
    # one iteration: the fused epilogue also applies the 1/||U|| scale of
    # the first iteration; none: nothing to fuse, the apply kernel runs
    mats, n, _ = _layout(SHAPES)
    a = Case(gpu, mats, n, 12)
    b = Case(gpu, mats, n, 12)
    hp = mhp(QUINTIC, steps=steps)
    M.muon_step(a.plan, a.params, a.grads, a.mom, a.ws, hp)
    M.muon_step(b.plan, b.params, b.grads, b.mom, b.ws, hp, b.out)
    torch.cuda.synchronize()
    assert torch.equal(a.params.view(torch.int16), b.params.view(torch.int16))
    assert torch.equal(a.mom, b.mom)


def test_stage_ns_apply_composes_like_the_step(gpu):
    mats, n, _ = _layout(SHAPES)
    a = Case(gpu, mats, n, 6)
    b = Case(gpu, mats, n, 6)
    hp = mhp(QUINTIC)
    M.muon_stage_momentum(a.plan, 0, a.grads, a.mom, a.ws, hp)
    for it in range(hp.ns_steps):
        for ph in (1, 2):
            M.muon_stage_ns_phase(a.plan, 0, a.ws, hp, it, ph)
        if it < hp.ns_steps - 1:
            M.muon_stage_ns_phase(a.plan, 0, a.ws, hp, it, 3)
    M.muon_stage_ns_apply(a.plan, 0, a.params, a.ws, hp)
    M.muon_step(b.plan, b.params, b.grads, b.mom, b.ws, hp, b.out)
    torch.cuda.synchronize()
    assert torch.equal(a.params.view(torch.int16), b.params.view(torch.int16))
    assert torch.equal(a.mom, b.mom)


def test_fused_step_over_waves_and_fallbacks(gpu):
    mats, n, _ = _layout(SHAPES)
    hp = mhp(QUINTIC, steps=3, scale_mode=1)
    # waves: a workspace cap that splits the matrices
    a = Case(gpu, mats, n, 7)
    cap = a.plan.workspace_bytes * 6 // 10   # one of the two large matrices per wave
    capped = M.muon_plan_create(mats, n, "bf16", "bf16", "bf16", cap)
    assert capped.info().n_waves > 1
    ws = capped.alloc_workspace(gpu)
    b = Case(gpu, mats, n, 7)
    M.muon_step(capped, a.params, a.grads, a.mom, ws, hp)
    M.muon_step(b.plan, b.params, b.grads, b.mom, b.ws, hp, b.out)
    torch.cuda.synchronize()
    assert torch.equal(a.params.view(torch.int16), b.params.view(torch.int16))
    # a parameter buffer 2 bytes off 16-byte alignment: the apply kernel runs
    base = torch.zeros(n + 1, dtype=BF16, device=gpu)
    c = Case(gpu, mats, n, 8)
    base[1:].copy_(c.params)
    d = Case(gpu, mats, n, 8)
    M.muon_step(c.plan, base[1:], c.grads, c.mom, c.ws, hp)
    M.muon_step(d.plan, d.params, d.grads, d.mom, d.ws, hp, d.out)
    torch.cuda.synchronize()
    assert torch.equal(base[1:].view(torch.int16), d.params.view(torch.int16))
    assert base[0].item() == 0.0
    # fp32 params: never fused
    e = Case(gpu, mats, n, 9, pdt="fp32")
    assert e.plan.info().fused_apply_mats == 0


def test_guard_skip_leaves_params_alone(gpu):
    mats, n, _ = _layout(SHAPES)
    a = Case(gpu, mats, n, 10)
    clip = torch.zeros(4, dtype=torch.int32, device=gpu)
    clip.view(torch.float32)[1] = 1.0   # scale
    clip[2] = 1                          # skip
    p0, m0 = a.params.clone(), a.mom.clone()
    M.muon_step(a.plan, a.params, a.grads, a.mom, a.ws, mhp(QUINTIC), clip=clip)
    torch.cuda.synchronize()
    assert torch.equal(a.params.view(torch.int16), p0.view(torch.int16))
    assert torch.equal(a.mom, m0)


def test_dense_stack_fused_full_size(gpu):
    """The dense d2048 x 16 stack as timed: every matrix fused, W bitwise
    the apply kernel's."""
    wl = W.workload("dense_d2048_l16")
    hp = mhp(QUINTIC)
    res = []
    for with_out in (False, True):
        inp = W.make_muon_inputs(wl, gpu, step=1)
        plan = M.muon_plan_create(wl.mats(), wl.muon_numel(), "bf16", "bf16", "bf16")
        assert plan.info().fused_apply_mats == 112
        ws = plan.alloc_workspace(gpu)
        out = torch.zeros(wl.muon_numel(), device=gpu) if with_out else None
        M.muon_step(plan, inp.params, inp.grads, inp.momentum, ws, hp, out)
        torch.cuda.synchronize()
        res.append(inp.params.view(torch.int16).clone())
        del inp, ws, out
        torch.cuda.empty_cache()
    assert torch.equal(res[0], res[1])


def test_one_plan_two_streams_concurrently(gpu):
    """A plan is immutable and shareable: two steps on two streams, each
    with its own workspace and buffers, running at the same time, give
    bitwise what each gives alone (no state hidden in the plan or library)."""
    mats, n, _ = _layout(SHAPES)
    hp = mhp(QUINTIC)
    ref = [Case(gpu, mats, n, 40 + k) for k in range(2)]
    for c in ref:
        M.muon_step(c.plan, c.params, c.grads, c.mom, c.ws, hp)
        torch.cuda.synchronize()
    run = [Case(gpu, mats, n, 40 + k) for k in range(2)]
    plan = run[0].plan                  # one plan for both streams
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for c, s in zip(run, streams):
        with torch.cuda.stream(s):
            M.muon_step(plan, c.params, c.grads, c.mom, c.ws, hp)
    torch.cuda.synchronize()
    for c, r in zip(run, ref):
        assert torch.equal(c.params.view(torch.int16), r.params.view(torch.int16))
        assert torch.equal(c.mom, r.mom)
