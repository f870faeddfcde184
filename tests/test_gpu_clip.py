"""GPU parity of MuonClip (muon_clip, through the C ABI) against the fp64
oracle in oracle/clip_oracle.py.

Tolerances:
  elements outside every block          bitwise unchanged
  blocks that are not clipped           bitwise unchanged
  clipped blocks                        every element within one storage
      ulp of the oracle's and at most 1e-4 of them differ: both sides
      compute gamma * w in fp64 and round it to fp32 (then bf16); gamma
      can differ in its last bits because the fp64 sums of squares are
      added in another order, which moves a product across a rounding
      boundary only rarely
  norms_out                             relative 1e-6 (fp32 of an fp64 norm)
  scales_out                            relative 1e-6 (fp32 of an fp64 gamma)
  recomputed max logit after the clip   relative 1e-5 of tau (fp32 params)
"""

import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as M
from muon_newton_schulz_amd import workloads as W
from oracle import clip_oracle as C
from oracle import muon_oracle as O

from test_gpu_adamw_states import _spacing
from test_gpu_parity import np64

pytestmark = pytest.mark.gpu

TORCH = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _layout():
    """Blocks of every kind, as (offset, rows, cols, ld, group): whole
    matrices over several chunks with ragged tails, head row blocks,
    strided column blocks (vector and scalar paths), one long row, a tiny
    block; gaps between them stay untouched."""
    t, o = [], 3
    t.append((o, 300, 257, 257, 0)); o += 300 * 257 + 5          # 3 chunks, scalar path
    o = (o + 7) // 8 * 8
    t.append((o, 256, 512, 512, 0)); o += 256 * 512 + 8          # 4 chunks, vector path
    for h in range(8):                                           # 512 x 256 W_q, 8 heads
        t.append((o + h * 64 * 256, 64, 256, 256, 0))
    o += 512 * 256 + 16
    for j in range(3):                                           # 128 x 192, 3 column blocks
        t.append((o + 64 * j, 128, 64, 192, 0))
    o += 128 * 192 + 1
    t.append((o, 1, 1000, 1000, 0)); o += 1000 + 2               # one row, odd offset
    t.append((o, 3, 5, 5, 0)); o += 15 + 3                       # tiny
    t.append((o, 40, 7, 9, 0)); o += 40 * 9 + 4                  # strided, scalar path
    return t, o


def _weights(targets, n, dtype, dev, seed):
    """N(0, 1) values, each block scaled differently so that one tau clips
    some blocks and not others."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    flat = torch.randn(n, generator=g, device=dev)
    for i, (off, rows, cols, ld, _) in enumerate(targets):
        idx = off + torch.arange(rows, device=dev)[:, None] * ld + torch.arange(cols, device=dev)
        flat[idx.reshape(-1)] *= 0.01 * (1.0 + (i % 5)) / (rows * cols) ** 0.5 * 30
    return flat.to(dtype)


def _check_flat(got, want, before, targets, gammas, dt):
    touched = np.zeros(got.size, bool)
    for t, g in zip(targets, gammas):
        idx, _ = C.block_view(before, t)
        touched[idx] = True
        if g == 1.0:
            assert np.array_equal(got[idx], before[idx])
    assert np.array_equal(got[~touched], before[~touched])
    ulp = (2.0 ** -23 * np.maximum(np.abs(got), np.abs(want))) if dt == "fp32" else \
        np.maximum(_spacing(got, dt), _spacing(want, dt))
    assert np.all(np.abs(got - want) <= ulp)
    assert np.count_nonzero(got != want) <= 1e-4 * max(touched.sum(), 1) + 1


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("shift", [0, 1])
def test_frobenius_clip_matches_oracle(gpu, dt, shift):
    # shift = 1 moves the whole buffer by one element: the scalar paths
    targets, n = _layout()
    base = _weights(targets, n + shift, TORCH[dt], gpu, 5)
    w = base[shift:]
    before = np64(w)
    norms = [C.frobenius_clip_factor(C.block_view(before, t)[1], 1.0)[0] for t in targets]
    tau = float(np.float32(np.median(norms)))
    plan = M.muon_clip_plan_create(targets, n, dt)
    no = torch.zeros(len(targets), device=gpu)
    so = torch.zeros(len(targets), device=gpu)
    M.muon_clip(plan, w, "frobenius", tau, norms_out=no, scales_out=so)
    torch.cuda.synchronize()
    want, rn, rg = C.muon_clip_flat(before, targets, C.MODE_FROBENIUS, tau, None, dt)
    assert 0 < sum(g < 1.0 for g in rg) < len(targets)
    np.testing.assert_allclose(np64(no), rn, rtol=1e-6)
    np.testing.assert_allclose(np64(so), rg, rtol=1e-6)
    _check_flat(np64(w), want, before, targets, rg, dt)
    # deterministic: the same input gives the same bits
    w2 = torch.tensor(before, device=gpu).to(TORCH[dt])
    M.muon_clip(plan, w2, "frobenius", tau)
    torch.cuda.synchronize()
    if shift == 0:
        assert torch.equal(w2, w)


def _attention(gpu, dt, layers, heads, d_head, d_model, seed):
    g = torch.Generator(device=gpu)
    g.manual_seed(seed)
    per = heads * d_head * d_model
    flat = torch.randn(2 * layers * per, generator=g, device=gpu).to(TORCH[dt])
    targets = []
    for l in range(layers):
        for h in range(heads):
            grp = l * heads + h
            q = 2 * l * per + h * d_head * d_model
            k = (2 * l + 1) * per + h * d_head * d_model
            targets.append((q, d_head, d_model, d_model, grp))
            targets.append((k, d_head, d_model, d_model, grp))
    return flat, targets


def test_max_logit_clip_matches_oracle(gpu):
    layers, heads, d_head, d_model = 2, 4, 64, 256
    flat, targets = _attention(gpu, "bf16", layers, heads, d_head, d_model, 7)
    tau = 100.0
    S = torch.tensor([50.0, 200.0, 100.0, 1e4, float("nan"), float("inf"), 300.0, -5.0],
                     device=gpu)
    before = np64(flat)
    plan = M.muon_clip_plan_create(targets, flat.numel(), "bf16", n_groups=layers * heads)
    assert plan.workspace_bytes > 0
    so = torch.zeros(len(targets), device=gpu)
    no = torch.full((len(targets),), -1.0, device=gpu)
    M.muon_clip(plan, flat, "max_logit", tau, max_logits=S, scales_out=so, norms_out=no)
    torch.cuda.synchronize()
    want, _, rg = C.muon_clip_flat(before, targets, C.MODE_MAX_LOGIT, tau,
                                   [float(x) for x in np64(S)], "bf16")
    assert [g < 1.0 for g in rg[::2]] == [False, True, False, True, False, False, True, False]
    np.testing.assert_allclose(np64(so), rg, rtol=1e-6)
    assert np.all(np64(no) == 0.0)
    _check_flat(np64(flat), want, before, targets, rg, "bf16")


def test_max_logit_clip_bounds_the_recomputed_logit(gpu):
    """After the clip, each clipped head's largest logit on the same queries
    and keys is tau (fp32 params): the property at any size."""
    layers, heads, d_head, d_model = 1, 4, 32, 128
    flat, targets = _attention(gpu, "fp32", layers, heads, d_head, d_model, 9)
    x = np.random.default_rng(3).standard_normal((24, d_model))
    per = heads * d_head * d_model
    wq = np64(flat[:per]).reshape(heads * d_head, d_model)
    wk = np64(flat[per:2 * per]).reshape(heads * d_head, d_model)
    S = [C.attention_max_logit(x, wq[h * d_head:(h + 1) * d_head], wk[h * d_head:(h + 1) * d_head])
         for h in range(heads)]
    tau = float(np.float32(np.median(S)))
    plan = M.muon_clip_plan_create(targets, flat.numel(), "fp32", n_groups=heads)
    M.muon_clip(plan, flat, "max_logit", tau,
                max_logits=torch.tensor(S, dtype=torch.float32, device=gpu))
    torch.cuda.synchronize()
    wq2 = np64(flat[:per]).reshape(wq.shape)
    wk2 = np64(flat[per:2 * per]).reshape(wk.shape)
    for h in range(heads):
        sl = slice(h * d_head, (h + 1) * d_head)
        s2 = C.attention_max_logit(x, wq2[sl], wk2[sl])
        s_in = float(np.float32(S[h]))
        if s_in > tau:
            assert abs(s2 - tau) <= 1e-5 * tau, (h, s2, tau)
        else:
            assert np.array_equal(wq2[sl], wq[sl]) and np.array_equal(wk2[sl], wk[sl])


def test_clip_edge_cases(gpu):
    # no targets: a no-op; a zero block and a NaN block are left alone
    w = torch.ones(100, dtype=torch.bfloat16, device=gpu)
    plan0 = M.muon_clip_plan_create([], 100, "bf16")
    assert plan0.workspace_bytes == 0
    M.muon_clip(plan0, w, "frobenius", 1.0)
    w[:10] = 0.0
    w[20] = float("nan")
    plan = M.muon_clip_plan_create([(0, 2, 5), (20, 1, 10), (40, 6, 10)], 100, "bf16")
    so = torch.zeros(3, device=gpu)
    no = torch.zeros(3, device=gpu)
    before = w.clone()
    M.muon_clip(plan, w, "frobenius", 1.0, norms_out=no, scales_out=so)
    torch.cuda.synchronize()
    assert np64(so).tolist() == [1.0, 1.0, pytest.approx(1.0 / 60 ** 0.5, rel=1e-6)]
    assert np64(no)[0] == 0.0 and np.isnan(np64(no)[1])
    assert torch.equal(w[:40].view(torch.int16), before[:40].view(torch.int16))  # NaN kept
    assert np.array_equal(np64(w[40:100]), O.bf16_round(np64(before[40:100]) / 60 ** 0.5))
    with pytest.raises(M.MuonError):
        M.muon_clip(plan, w, "frobenius", 0.0)
    with pytest.raises(M.MuonError):
        M.muon_clip(plan, w, "max_logit", 1.0, max_logits=torch.ones(1, device=gpu))


def test_dense_stack_qk_clip_full_size(gpu):
    """Frobenius clip of every W_q and W_k of the dense d2048 x 16 stack (the
    first two 2048 x 2048 matrices of each layer) on the generated weights:
    the norms against the oracle for all 32, the clipped values of two
    sampled matrices element by element."""
    wl = W.workload("dense_d2048_l16")
    inp = W.make_muon_inputs(wl, gpu, step=1)
    mats = wl.mats()
    qk = [m for m in mats if m[1] == m[2] == 2048]
    qk = [qk[4 * l + j] for l in range(16) for j in (0, 1)]
    targets = [(o, r, c, c, 0) for (o, r, c) in qk]
    w = inp.params
    norms = []
    for (o, r, c, _, _) in targets:
        blk = np64(w[o:o + r * c])
        norms.append(float(np.sqrt(np.dot(blk, blk))))
    tau = float(np.float32(np.median(norms)))
    plan = M.muon_clip_plan_create(targets, w.numel(), "bf16")
    sample = [targets[3], targets[20]]
    before = [np64(w[o:o + r * c]) for (o, r, c, _, _) in sample]
    no = torch.zeros(len(targets), device=gpu)
    so = torch.zeros(len(targets), device=gpu)
    M.muon_clip(plan, w, "frobenius", tau, norms_out=no, scales_out=so)
    torch.cuda.synchronize()
    np.testing.assert_allclose(np64(no), norms, rtol=1e-6)
    for (o, r, c, ld, g), b in zip(sample, before):
        local = (0, r, c, ld, g)
        want, _, rg = C.muon_clip_flat(b, [local], C.MODE_FROBENIUS, tau, None, "bf16")
        _check_flat(np64(w[o:o + r * c]), want, b, [local], rg, "bf16")
