"""Parity at the largest shapes, against the fp64 oracle: 8192-sided
matrices (the largest Muon matrices of the ragged workload) on the tiled
engine, vectors at the longest side a plan accepts, AdamW over the
ragged workload's 1.17e9-element embedding and past 2^31 elements, and the
gradient-norm and state-statistics reductions past 2^31 elements (closed
forms: constant buffers).

The oracle cannot run NS on an 8192 x 8192 matrix in seconds, so the big
matrices get an embedded input: the gradient is zero outside a scattered
set of rows R and columns C, and the momentum starts at zero.  With P and Q
the 0/1 matrices that select R and C (P P^T = I, Q Q^T = I), the normalised
input is X = P^T B Q for the compressed block B = G[R][:, C], so
X X^T = P^T (B B^T) P, and every NS iterate is P^T (iterate of B) Q: the
result on R x C is the NS of B alone, and exactly zero elsewhere.  The
Frobenius norm of X is that of B.  Scale mode 2 (s = 1) keeps the update of
W independent of the matrix's dims, so the oracle's whole step on the
compressed block gives the expected W, M and O on R x C.  Rows outside R
see a zero gradient: the oracle's step on a few of them, at full width,
gives their W (weight decay only).

Tolerances as in the other parity tests: O relative 1e-2 (bf16 NS) or 1e-4
(fp32 NS), M 2e-6, W 1e-2 (bf16 params) on the block; outside the block O
and M exactly zero and W within one bf16 ulp of the oracle's rounded value
(both sides round their own product to nearest).
"""

import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as M
from oracle import muon_oracle as O

from test_gpu_adamw_states import _spacing
from test_gpu_parity import QUINTIC, TOL_O, _flat, mhp, np64, ohp, rel

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _embedded_case(gpu, shapes, ns_dtype, seed):
    """Flat buffers for ``shapes`` with a gradient supported on scattered
    rows R x columns C of each matrix (150-260 rows, 200-330 columns)."""
    rng = np.random.default_rng(seed)
    g = torch.Generator(device=gpu)
    g.manual_seed(seed)
    mats, n = _flat(shapes)
    params = (torch.randn(n, generator=g, device=gpu) * 0.02).to(BF16)
    grads = torch.zeros(n, dtype=BF16, device=gpu)
    supports = []
    for (o, r, c) in mats:
        R = np.sort(rng.choice(r, size=int(rng.integers(150, 261)), replace=False))
        C = np.sort(rng.choice(c, size=int(rng.integers(200, 331)), replace=False))
        idx = (o + torch.tensor(R, device=gpu)[:, None] * c
               + torch.tensor(C, device=gpu)[None, :]).reshape(-1)
        grads[idx] = (torch.randn(idx.numel(), generator=g, device=gpu) * 0.02).to(BF16)
        supports.append((R, C, idx))
    mom = torch.zeros(n, device=gpu)
    out = torch.full((n,), 7.0, device=gpu)
    plan = M.muon_plan_create(mats, n, "bf16", "bf16", ns_dtype)
    return mats, params, grads, mom, out, plan, supports


@pytest.mark.parametrize("shapes,ns_dtype", [
    # square at 8192; tall off the 64 grid; wide with an 8192-long K
    ([(8192, 8192), (8229, 3001), (1000, 8192)], "bf16"),
    ([(8192, 8192)], "fp32"),
])
def test_embedded_block_at_8192(gpu, shapes, ns_dtype):
    mats, params, grads, mom, out, plan, supports = _embedded_case(gpu, shapes, ns_dtype, 31)
    hp = mhp(QUINTIC, scale_mode=2)
    ws = plan.alloc_workspace(gpu)
    rng = np.random.default_rng(7)
    before = []
    for (o, r, c), (R, C, idx) in zip(mats, supports):
        outside = np.setdiff1d(np.arange(r), R)
        rows = np.sort(rng.choice(outside, size=4, replace=False))
        ridx = (o + torch.tensor(rows, device=gpu)[:, None] * c
                + torch.arange(c, device=gpu)[None, :]).reshape(-1)
        before.append((np64(params[idx]).reshape(len(R), len(C)),
                       np64(grads[idx]).reshape(len(R), len(C)),
                       rows, ridx, np64(params[ridx]).reshape(len(rows), c)))
    M.muon_step(plan, params, grads, mom, ws, hp, out)
    torch.cuda.synchronize()
    for (o, r, c), (R, C, idx), (Wb, Gb, rows, ridx, Wr) in zip(mats, supports, before):
        case = (r, c, ns_dtype)
        # the block against the oracle's step on the compressed block
        Wn, Mn, On = O.muon_matrix_math(Wb, Gb, np.zeros_like(Gb), ohp(hp))
        assert rel(np64(out[idx]).reshape(Wb.shape), On) <= TOL_O[ns_dtype], case
        assert rel(np64(mom[idx]), O.fp32_round(Mn).ravel()) <= 2e-6, case
        assert rel(np64(params[idx]), O.bf16_round(Wn).ravel()) <= 1e-2, case
        # outside the block: O and M exactly zero
        o_mat = out[o:o + r * c].clone()
        m_mat = mom[o:o + r * c].clone()
        o_mat[idx - o] = 0.0
        m_mat[idx - o] = 0.0
        assert int(torch.count_nonzero(o_mat)) == 0, case
        assert int(torch.count_nonzero(m_mat)) == 0, case
        # whole rows outside R: weight decay only
        Wr_n, _, Or = O.muon_matrix_math(Wr, np.zeros_like(Wr), np.zeros_like(Wr), ohp(hp))
        assert not Or.any()
        want = O.bf16_round(Wr_n).ravel()
        got = np64(params[ridx])
        assert np.all(np.abs(got - want) <= _spacing(want, "bf16")), case


@pytest.mark.parametrize("shape", [(1, 16383 * 256), (16383 * 256, 1)])
def test_vector_at_the_longest_side(gpu, shape):
    # the longest side a bf16-NS plan accepts: phase 1 runs one tile over a
    # 4194048-long K, phase 3 16383 tiles of one row
    r, c = shape
    n = r * c + 5
    g = torch.Generator(device=gpu)
    g.manual_seed(3)
    params = (torch.randn(n, generator=g, device=gpu) * 0.02).to(BF16)
    grads = (torch.randn(n, generator=g, device=gpu) * 0.02).to(BF16)
    mom = torch.zeros(n, device=gpu)
    out = torch.full((n,), 7.0, device=gpu)
    mats = [(3, r, c)]
    plan = M.muon_plan_create(mats, n, "bf16", "bf16", "bf16")
    ws = plan.alloc_workspace(gpu)
    hp = mhp(QUINTIC)
    W0, G0 = np64(params[3:3 + r * c]), np64(grads[3:3 + r * c])
    M.muon_step(plan, params, grads, mom, ws, hp, out)
    torch.cuda.synchronize()
    Wn, Mn, On = O.muon_matrix_math(W0.reshape(r, c), G0.reshape(r, c),
                                    np.zeros((r, c)), ohp(hp))
    assert rel(np64(out[3:3 + r * c]), On.ravel()) <= TOL_O["bf16"]
    assert rel(np64(mom[3:3 + r * c]), O.fp32_round(Mn).ravel()) <= 2e-6
    assert rel(np64(params[3:3 + r * c]), O.bf16_round(Wn).ravel()) <= 1e-2
    # untouched head and tail
    assert np.all(np64(out[:3]) == 7.0) and np.all(np64(out[3 + r * c:]) == 7.0)
    del ws
    torch.cuda.empty_cache()


def _adam_check(p_got, master_got, m_got, v_got, p0, m0, g, hp, pdt):
    """Oracle step on sampled elements; tolerances as for the other AdamW
    parity tests (2e-6 relative on the states and master, bf16 params the
    cast of the GPU's own master)."""
    from test_gpu_parity import adam_oracle_run
    pr, mr_, er, vr = adam_oracle_run(p0, m0, [g], hp, pdt)
    assert rel(v_got, vr) <= 2e-6 and rel(m_got, er) <= 2e-6
    if master_got is not None:
        assert rel(master_got, mr_) <= 2e-6
        np.testing.assert_array_equal(p_got, O.bf16_round(master_got))
    else:
        assert rel(p_got, pr) <= 2e-6


def test_adamw_ragged_embedding_group_full_size(gpu):
    # the 163840 x 7168 embedding of the ragged workload (1.17e9 bf16
    # params, fp32 master): head, middle and tail sampled
    from muon_newton_schulz_amd import workloads as W
    wl = W.workload("ragged_500")
    gi = max(range(len(wl.adam)), key=lambda i: wl.adam[i].numel)
    grp = wl.adam[gi]
    assert grp.numel == 163840 * 7168 and grp.master
    a = W.make_adam_inputs(wl, gi, device=gpu)
    g = W.make_adam_grad(wl, gi, 1, device=gpu)
    n = grp.numel
    samples = [slice(0, 4099), slice(n // 2 - 3001, n // 2 + 3001), slice(n - 4099, n)]
    before = [(np64(a.param[s]), np64(a.master[s]), np64(g[s])) for s in samples]
    M.adamw_step(a.param, a.master, g, a.exp_avg, a.exp_avg_sq, wl.adam_hp, 1)
    torch.cuda.synchronize()
    for s, (p0, m0, gg) in zip(samples, before):
        _adam_check(np64(a.param[s]), np64(a.master[s]), np64(a.exp_avg[s]),
                    np64(a.exp_avg_sq[s]), p0, m0, gg, wl.adam_hp, "bf16")
    del a, g
    torch.cuda.empty_cache()


def test_adamw_past_2_31_elements(gpu):
    # fp32 params without master, 2^31 + 12345 elements: the kernel's
    # element indices pass 2^31 (64-bit indexing), sampled around it and at
    # the tail
    from muon_newton_schulz_amd import workloads as W
    n = (1 << 31) + 12345
    gen = torch.Generator(device=gpu)
    gen.manual_seed(23)
    p = torch.randn(n, generator=gen, device=gpu)
    g = torch.randn(n, generator=gen, device=gpu).to(torch.bfloat16)
    m = torch.zeros(n, device=gpu)
    v = torch.zeros(n, device=gpu)
    hp = W.AdamWHParams()
    samples = [slice(0, 1000), slice((1 << 31) - 2000, (1 << 31) + 2000), slice(n - 1000, n)]
    before = [(np64(p[s]), np64(g[s])) for s in samples]
    M.adamw_step(p, None, g, m, v, hp, 1)
    torch.cuda.synchronize()
    for s, (p0, gg) in zip(samples, before):
        _adam_check(np64(p[s]), None, np64(m[s]), np64(v[s]), p0, None, gg, hp, "fp32")
    del p, g, m, v
    torch.cuda.empty_cache()


def test_guard_reductions_past_2_31_elements(gpu):
    # closed forms past 2^31 elements: the global norm of a constant bf16
    # buffer is c sqrt(n) (the fp64 sum of the c^2 is exact); the statistics
    # of a constant fp32 buffer with one NaN and one +Inf beyond index 2^31
    n = (1 << 31) + 7
    g = torch.full((n,), 0.5, dtype=BF16, device=gpu)
    st = M.read_clip_state(M.grad_norm_clip([g], 1.0))
    assert abs(st["norm"] - 0.5 * n ** 0.5) <= 1e-7 * 0.5 * n ** 0.5
    assert not st["skip"]
    del g
    x = torch.full((n,), 1.5, device=gpu)
    x[(1 << 31) + 3] = float("nan")
    x[(1 << 31) + 5] = float("inf")
    s = M.read_state_stats(M.state_stats(x))
    assert s["count"] == n - 2 and s["nonfinite"] == 2
    assert s["mean"] == 1.5 and s["var"] == 0.0
    assert s["min"] == s["max"] == s["absmax"] == 1.5
    del x
    torch.cuda.empty_cache()
