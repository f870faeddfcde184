"""Holding each XCD's tile rounds together (NS phases 1 and 2, where the
plan finds a round's tiles cost much the same) is a timing device: the
results must be bitwise those of the free-running walk, in a plain step and
with two steps running at once on two streams, where the workgroups of one
kernel may wait for those of a group that is not yet resident (the wait is
bounded).  One matrix is also checked against the fp64 oracle."""

import pytest
import torch

from test_gpu_parity import QUINTIC, Setup, check_muon_step, mhp

pytestmark = pytest.mark.gpu

SIDE = 2304  # 9 tiles per side: diagonal tiles last, uniform rounds
N_MATS = 24  # 24 x 45 triangle tiles: 5 rounds of 256, one hold


def _mats():
    return [(k * SIDE * SIDE, SIDE, SIDE) for k in range(N_MATS)]


def _pair(gpu, seed):
    held = Setup(_mats(), N_MATS * SIDE * SIDE, "bf16", "bf16", "bf16", gpu, seed=seed)
    free = Setup(_mats(), N_MATS * SIDE * SIDE, "bf16", "bf16", "bf16", gpu, seed=seed,
                 free_rounds=True)
    assert held.plan.info().round_sync_phases == 0b11
    assert free.plan.info().round_sync_phases == 0
    return held, free


def test_held_rounds_match_free_rounds_bitwise(gpu):
    held, free = _pair(gpu, 5)
    hp = mhp(QUINTIC)
    # one matrix against the oracle, the step itself on all of them
    check_muon_step(held, hp, only=[N_MATS - 1])
    free.step(hp)
    torch.cuda.synchronize()
    assert torch.equal(held.params, free.params)
    assert torch.equal(held.mom, free.mom)
    assert torch.equal(held.out, free.out)


def test_held_rounds_with_two_steps_at_once(gpu):
    a, ref_a = _pair(gpu, 11)
    b, ref_b = _pair(gpu, 12)
    hp = mhp(QUINTIC)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(2):  # the held plans step side by side, the free ones alone
        with torch.cuda.stream(s1):
            a.step(hp)
        with torch.cuda.stream(s2):
            b.step(hp)
        torch.cuda.synchronize()
        ref_a.step(hp)
        torch.cuda.synchronize()
        ref_b.step(hp)
        torch.cuda.synchronize()
    for s, r in ((a, ref_a), (b, ref_b)):
        assert torch.equal(s.params, r.params)
        assert torch.equal(s.mom, r.mom)
        assert torch.equal(s.out, r.out)
