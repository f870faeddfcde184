"""The Python binding checks every tensor before its address crosses the C
ABI (which sees only pointers): GPU residency, contiguity, element counts
against the plan, dtypes.  CPU-only: a stand-in tensor reports what the
checks read, and every case must fail before any library call."""

import pytest
import torch

import muon_newton_schulz_amd as M


class FakeGpuTensor:
    """Answers the questions the binding asks of a tensor."""

    def __init__(self, n, dtype=torch.bfloat16, contiguous=True, cuda=True):
        self._n, self.dtype, self._c, self.is_cuda = n, dtype, contiguous, cuda
        self.device = torch.device("cpu")

    def numel(self):
        return self._n

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        raise AssertionError("the address must not be taken before the checks pass")


def _plan(n=1000):
    return M.MuonPlan(0, 4096, 1, flat_numel=n, param_dtype=M.MUON_DTYPE_BF16,
                      grad_dtype=M.MUON_DTYPE_BF16)


def _err(fn, status):
    with pytest.raises(M.MuonError) as e:
        fn()
    assert e.value.status == status, e.value


def test_muon_step_checks_buffers_against_the_plan():
    plan = _plan()
    P, G = FakeGpuTensor(1000), FakeGpuTensor(1000)
    Mo, W = FakeGpuTensor(1000, torch.float32), FakeGpuTensor(4096, torch.uint8)
    hp = M.MuonHParamsC()
    _err(lambda: M.muon_step(plan, FakeGpuTensor(999), G, Mo, W, hp), M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.muon_step(plan, P, FakeGpuTensor(1000, torch.float32), Mo, W, hp),
         M.MUON_ERR_BAD_DTYPE)
    _err(lambda: M.muon_step(plan, P, G, FakeGpuTensor(1000, torch.bfloat16), W, hp),
         M.MUON_ERR_BAD_DTYPE)
    _err(lambda: M.muon_step(plan, P, G, Mo, W, hp, out_update=FakeGpuTensor(10, torch.float32)),
         M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.muon_step(plan, FakeGpuTensor(1000, contiguous=False), G, Mo, W, hp),
         M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.muon_step(plan, P, G, Mo, torch.empty(4096, dtype=torch.uint8), hp),
         M.MUON_ERR_INVALID_ARG)  # workspace on the host
    _err(lambda: M.muon_stage_apply(plan, 0, FakeGpuTensor(5), W, hp), M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.muon_stage_ns_apply(plan, 0, FakeGpuTensor(5), W, hp), M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.muon_stage_ns_apply(plan, 0, FakeGpuTensor(1000, torch.float32), W, hp),
         M.MUON_ERR_BAD_DTYPE)
    _err(lambda: M.muon_stage_momentum(plan, 0, G, FakeGpuTensor(999, torch.float32), W, hp),
         M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.muon_stage_export_x(plan, 0, W, 0, FakeGpuTensor(999, torch.float32)),
         M.MUON_ERR_INVALID_ARG)


def test_adamw_and_guard_check_their_tensors():
    hp = M.AdamWHParamsC(0.01, 0.9, 0.95, 1e-8, 0.1)
    p = FakeGpuTensor(100, torch.float32)
    g = FakeGpuTensor(100)
    m, v = FakeGpuTensor(100, torch.float32), FakeGpuTensor(100, torch.float32)
    _err(lambda: M.adamw_step(p, None, g, FakeGpuTensor(100, torch.float32, contiguous=False), v,
                              hp, 1), M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.adamw_step(p, None, g, m, FakeGpuTensor(99, torch.float32), hp, 1),
         M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.adamw_step(p, None, torch.zeros(100), m, v, hp, 1), M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.grad_norm_clip([g, FakeGpuTensor(10, contiguous=False)], 1.0,
                                  out=FakeGpuTensor(16, torch.uint8)), M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.grad_norm_clip([g], 1.0, out=FakeGpuTensor(8, torch.uint8)),
         M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.state_stats(FakeGpuTensor(10), out=FakeGpuTensor(56, torch.uint8)),
         M.MUON_ERR_BAD_DTYPE)
    _err(lambda: M.state_stats(FakeGpuTensor(10, torch.float32), out=FakeGpuTensor(8, torch.uint8)),
         M.MUON_ERR_INVALID_ARG)


def test_muon_clip_checks_its_tensors():
    plan = M.MuonClipPlan(0, 64, 3, 2, 1000, M.MUON_DTYPE_BF16)
    w = FakeGpuTensor(1000)
    _err(lambda: M.muon_clip(plan, FakeGpuTensor(999), "frobenius", 1.0), M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.muon_clip(plan, FakeGpuTensor(1000, torch.float32), "frobenius", 1.0),
         M.MUON_ERR_BAD_DTYPE)
    _err(lambda: M.muon_clip(plan, w, "max_logit", 1.0, max_logits=FakeGpuTensor(1, torch.float32)),
         M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.muon_clip(plan, w, "max_logit", 1.0, max_logits=None), M.MUON_ERR_INVALID_ARG)
    _err(lambda: M.muon_clip(plan, w, "frobenius", 1.0, workspace=FakeGpuTensor(64, torch.uint8),
                             norms_out=FakeGpuTensor(2, torch.float32)), M.MUON_ERR_INVALID_ARG)
    plan.handle = 0  # nothing to destroy
