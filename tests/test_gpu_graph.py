"""The optimizer step captured in a HIP graph: the library's steps enqueue
kernels only (no allocation, no memset, no host synchronisation), so a
caller can capture one whole step -- gradient-norm clip, Muon over small
(fused) and tiled matrices, with the update applied by its own kernel or by
the last NS phase, AdamW -- and replay it.  Every replay must be
bitwise the eager step from the same state; eager work and host
synchronisation run between the replays.  AdamW's step count and every
hyper-parameter are fixed at capture, so the eager reference uses the same
values each step."""

import pytest
import torch

import muon_newton_schulz_amd as M
from muon_newton_schulz_amd import workloads as W

from test_gpu_parity import QUINTIC, Setup, mhp

pytestmark = pytest.mark.gpu


class State:
    def __init__(self, gpu, seed):
        # offsets on 8-element boundaries: the tiled (300, 520), (520, 300)
        # and (520, 296) take the fused update, (520, 300) with its rows
        # realigned onto the 8-element grid (cols % 8 != 0)
        mats, o = [], 8
        for r, c in [(128, 256), (96, 200), (300, 520), (520, 300), (64, 64), (520, 296)]:
            mats.append((o, r, c))
            o = (o + r * c + 7) // 8 * 8 + 8
        self.s = Setup(mats, o, "bf16", "bf16", "bf16", gpu, seed=seed)
        g = torch.Generator(device=gpu)
        g.manual_seed(seed + 1)
        n = 5000
        self.ap = (torch.randn(n, generator=g, device=gpu) * 0.02).to(torch.bfloat16)
        self.am = self.ap.float()
        self.ag = (torch.randn(n, generator=g, device=gpu) * 0.02).to(torch.bfloat16)
        self.m = torch.zeros(n, device=gpu)
        self.v = torch.zeros(n, device=gpu)
        self.clip = torch.zeros(16, dtype=torch.uint8, device=gpu)
        self.clip_ws = torch.empty(max(8, M.grad_norm_clip_workspace_size(2)), dtype=torch.uint8,
                                   device=gpu)

    def step(self, hp, ahp, with_out=True):
        s = self.s
        M.grad_norm_clip([s.grads, self.ag], 1.0, out=self.clip, workspace=self.clip_ws)
        # without out_update, the last NS phase applies the update itself
        M.muon_step(s.plan, s.params, s.grads, s.mom, s.ws, hp, s.out if with_out else None,
                    clip=self.clip)
        M.adamw_step(self.ap, self.am, self.ag, self.m, self.v, ahp, 1, clip=self.clip)

    def tensors(self):
        s = self.s
        return [s.params, s.mom, s.out, self.ap, self.am, self.m, self.v, self.clip]


@pytest.mark.parametrize("with_out", [True, False])
def test_captured_step_replays_bitwise(gpu, with_out):
    hp, ahp = mhp(QUINTIC), W.AdamWHParams()
    eager = State(gpu, 21)
    assert eager.s.plan.info().small_mats == 3
    assert eager.s.plan.info().fused_apply_mats == 3
    ref = []
    for _ in range(3):
        eager.step(hp, ahp, with_out)
        torch.cuda.synchronize()
        ref.append([t.clone() for t in eager.tensors()])

    cap = State(gpu, 21)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    snapshot = [t.clone() for t in cap.tensors()]
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            cap.step(hp, ahp, with_out)
    torch.cuda.synchronize()
    # capture does not run the work: restore the starting state anyway
    for t, s0 in zip(cap.tensors(), snapshot):
        t.copy_(s0)
    torch.cuda.synchronize()
    gen = torch.Generator(device=gpu)
    gen.manual_seed(99)
    for k in range(3):
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, generator=gen, device=gpu).sum()  # eager work between replays
        torch.cuda.synchronize()
        del junk
        for a, b in zip(cap.tensors(), ref[k]):
            assert torch.equal(a, b), k
