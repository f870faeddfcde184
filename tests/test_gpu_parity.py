"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (relative Frobenius norm per tensor, ||gpu - ref|| / ||ref||):
  O (orthogonalised update)  bf16 NS <= 1e-2, fp32 NS <= 1e-4
  momentum M, AdamW master/m/v  <= 2e-6
  W with bf16 params <= 1e-2 (one bf16 rounding of a value that differs by
    the NS error); W with fp32 params: lr*s*||dO|| / ||W||, derived per case.
Inputs come from the seeded generators in muon_newton_schulz_amd.workloads;
the oracle sees the same input values, converted exactly to float64.
"""

import math

import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as M
from muon_newton_schulz_amd import workloads as W
from oracle import muon_oracle as O

pytestmark = pytest.mark.gpu

CUBIC = W.CUBIC
QUINTIC = W.QUINTIC
TOL_O = {"bf16": 1e-2, "fp32": 1e-4}


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _gen(dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return g


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def mhp(coef=CUBIC, steps=5, **kw):
    hp = W.MuonHParams(ns_a=coef[0], ns_b=coef[1], ns_c=coef[2], ns_steps=steps)
    for k, v in kw.items():
        setattr(hp, k, v)
    return hp


def ohp(hp):
    return O.MuonHP(lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                    nesterov=hp.nesterov, ns_a=hp.ns_a, ns_b=hp.ns_b, ns_c=hp.ns_c,
                    ns_steps=hp.ns_steps, eps=hp.eps, scale_mode=hp.scale_mode,
                    rms_target=hp.rms_target)


class Setup:
    """Flat buffers + plan + workspace for a list of (offset, rows, cols)."""

    def __init__(self, mats, n, param_dtype, grad_dtype, ns_dtype, dev, seed=0,
                 w_std=1.0, g_std=1.0, cap=0, sentinel=True, tiled_only=False,
                 whole_tiles=False, free_rounds=False):
        self.mats, self.n = mats, n
        self.param_dtype, self.ns_dtype = param_dtype, ns_dtype
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        fill = 7.0 if sentinel else 0.0
        self.params = torch.full((n,), fill, dtype=W.TORCH_DTYPE[param_dtype], device=dev)
        self.grads = torch.full((n,), fill, dtype=W.TORCH_DTYPE[grad_dtype], device=dev)
        self.mom = torch.full((n,), fill, dtype=torch.float32, device=dev)
        for (o, r, c) in mats:
            self.params[o:o + r * c] = (torch.randn(r * c, generator=g, device=dev) * w_std).to(
                self.params.dtype)
            self.grads[o:o + r * c] = (torch.randn(r * c, generator=g, device=dev) * g_std).to(
                self.grads.dtype)
            self.mom[o:o + r * c] = 0.0
        self.plan = M.muon_plan_create(mats, n, param_dtype, grad_dtype, ns_dtype, cap,
                                       tiled_only=tiled_only, whole_tiles=whole_tiles,
                                       free_rounds=free_rounds)
        self.ws = self.plan.alloc_workspace(dev)
        self.out = torch.full((n,), fill, dtype=torch.float32, device=dev)

    def step(self, hp):
        M.muon_step(self.plan, self.params, self.grads, self.mom, self.ws, hp, self.out)

    def snapshot(self):
        return np64(self.params), np64(self.grads), np64(self.mom)


def check_muon_step(s: Setup, hp, tol_w=None, only=None):
    P0, G0, M0 = s.snapshot()
    s.step(hp)
    torch.cuda.synchronize()
    P1, M1, Og = np64(s.params), np64(s.mom), np64(s.out)
    Pr, Mr, outs = O.muon_step_flat(P0, G0, M0, s.mats, ohp(hp), s.param_dtype, only=only)
    idx = range(len(s.mats)) if only is None else only
    worst = {"O": 0.0, "M": 0.0, "W": 0.0}
    for i in idx:
        o, r, c = s.mats[i]
        sl = slice(o, o + r * c)
        eo = rel(Og[sl].reshape(r, c), outs[i])
        em = rel(M1[sl], Mr[sl])
        ew = rel(P1[sl], Pr[sl])
        assert eo <= TOL_O[s.ns_dtype], (i, r, c, "O", eo)
        assert em <= 2e-6, (i, r, c, "M", em)
        tw = tol_w if tol_w is not None else (1e-2 if s.param_dtype == "bf16" else 1e-4)
        assert ew <= tw, (i, r, c, "W", ew)
        worst = {k: max(worst[k], v) for k, v in (("O", eo), ("M", em), ("W", ew))}
    if only is None:
        covered = np.zeros(s.n, bool)
        for (o, r, c) in s.mats:
            covered[o:o + r * c] = True
        assert np.all(P1[~covered] == P0[~covered])
        assert np.all(M1[~covered] == M0[~covered])
        assert np.all(np64(s.out)[~covered] == 7.0)
    return worst


# ---------------------------------------------------------------- AdamW


def adam_oracle_run(p, master, g_list, hp, pdt, t0=1):
    th = master if master is not None else p
    m = np.zeros_like(th)
    v = np.zeros_like(th)
    out_p, out_master = p, master
    for k, g in enumerate(g_list):
        out_p, out_master, m, v = O.adamw_step_stored(out_p, out_master, g, m, v,
                                                      O.AdamWHP(hp.lr, hp.beta1, hp.beta2,
                                                                hp.eps, hp.weight_decay),
                                                      t0 + k, pdt)
    return out_p, out_master, m, v


def test_adamw_fp32_vector_ten_steps(gpu):
    wl = W.workload("single_fp32_128x256")
    a = W.make_adam_inputs(wl, 0, device=gpu)
    p0 = np64(a.param)
    grads = [W.make_adam_grad(wl, 0, t, device=gpu) for t in range(1, 11)]
    for t, g in enumerate(grads, 1):
        M.adamw_step(a.param, None, g, a.exp_avg, a.exp_avg_sq, wl.adam_hp, t)
    torch.cuda.synchronize()
    pr, _, mr, vr = adam_oracle_run(p0, None, [np64(g) for g in grads], wl.adam_hp, "fp32")
    assert rel(np64(a.param), pr) <= 2e-6
    assert rel(np64(a.exp_avg), mr) <= 2e-6
    assert rel(np64(a.exp_avg_sq), vr) <= 2e-6


def test_adamw_bf16_master_dense_groups_sampled(gpu):
    wl = W.workload("dense_d2048_l16")
    for gi, grp in enumerate(wl.adam):
        a = W.make_adam_inputs(wl, gi, device=gpu)
        n = grp.numel
        samples = [slice(0, min(n, 65536)), slice(n // 2 - 4097, n // 2 + 4097),
                   slice(max(0, n - 1001), n)]
        p0 = [np64(a.param[s]) for s in samples]
        m0 = [np64(a.master[s]) for s in samples]
        gs = []
        for t in (1, 2):
            g = W.make_adam_grad(wl, gi, t, device=gpu)
            gs.append([np64(g[s]) for s in samples])
            M.adamw_step(a.param, a.master, g, a.exp_avg, a.exp_avg_sq, wl.adam_hp, t)
        torch.cuda.synchronize()
        for k, s in enumerate(samples):
            pr, mr_, er, vr = adam_oracle_run(p0[k], m0[k], [gs[0][k], gs[1][k]], wl.adam_hp,
                                              "bf16")
            master = np64(a.master[s])
            assert rel(master, mr_) <= 2e-6, (grp.name, k)
            assert rel(np64(a.exp_avg[s]), er) <= 2e-6
            assert rel(np64(a.exp_avg_sq[s]), vr) <= 2e-6
            # bf16 param is the RNE cast of the GPU's own fp32 master ...
            np.testing.assert_array_equal(np64(a.param[s]), O.bf16_round(master))
            # ... and within one bf16 ulp of the oracle's
            ulp = np.maximum(np.abs(pr), 1e-30) * 2.0 ** -7
            assert np.all(np.abs(np64(a.param[s]) - pr) <= ulp * 1.01)


@pytest.mark.parametrize("n,off", [(1001, 1), (3, 0), (4099, 3), (1, 0), (1001, 0), (4101, 8)])
def test_adamw_unaligned_and_tails(gpu, n, off):
    g_ = torch.Generator(device=gpu)
    g_.manual_seed(n + off)
    base_p = torch.randn(n + 8, generator=g_, device=gpu)
    base_g = torch.randn(n + 8, generator=g_, device=gpu).to(torch.bfloat16)
    master = base_p[off:off + n].clone() if off == 0 else base_p[off:off + n]
    p = master.to(torch.bfloat16)
    pbuf = torch.zeros(n + 8, dtype=torch.bfloat16, device=gpu)
    pbuf[off:off + n] = p
    m = torch.zeros(n + 8, device=gpu)
    v = torch.zeros(n + 8, device=gpu)
    hp = W.AdamWHParams()
    m0 = np64(master)
    gg = np64(base_g[off:off + n])
    M.adamw_step(pbuf[off:off + n], master, base_g[off:off + n], m[off:off + n], v[off:off + n],
                 hp, 1)
    torch.cuda.synchronize()
    pr, mr_, er, vr = adam_oracle_run(O.bf16_round(m0), m0, [gg], hp, "bf16")
    assert rel(np64(master), mr_) <= 2e-6
    assert rel(np64(m[off:off + n]), er) <= 2e-6
    assert rel(np64(v[off:off + n]), vr) <= 2e-6
    assert np.all(np64(m[:off]) == 0) and np.all(np64(m[off + n:]) == 0)
    assert np.all(np64(pbuf[:off]) == 0) and np.all(np64(pbuf[off + n:]) == 0)


# ---------------------------------------------------------------- Muon, small


@pytest.mark.parametrize("ns_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("coef", [CUBIC, QUINTIC])
def test_muon_single_fp32_matrix_ten_steps(gpu, ns_dtype, coef):
    # 128x256 fp32 matrix, zero momentum, mu 0.95 Nesterov, 5 NS steps,
    # lr 0.02, wd 0.1, fresh gradients every step; checked every step
    # against the oracle started from the GPU's state.  fp32 W: the NS error
    # moves W by lr*s*||dO|| ~ 0.02*3.2*tol_O*||O|| with ||O|| <= sqrt(128),
    # ||W|| ~ 181, i.e. <= 4e-5 (bf16 NS) or 4e-7 (fp32 NS) relative.
    wl = W.workload("single_fp32_128x256")
    hp = mhp(coef)
    s = Setup(wl.mats(), wl.muon_numel(), "fp32", "fp32", ns_dtype, gpu, sentinel=False)
    s.params.copy_(W.make_muon_inputs(wl, gpu).params)
    tol_w = 4e-5 if ns_dtype == "bf16" else 1e-6
    for step in range(1, 11):
        W.make_muon_grads(wl, step, gpu, out=s.grads)
        check_muon_step(s, hp, tol_w=tol_w)


EDGE_SHAPES = [(1, 300), (300, 1), (63, 65), (65, 63), (129, 257), (257, 129), (256, 256),
               (1, 1), (17, 1409), (2, 2), (511, 513)]


def _flat(shapes, gap=3):
    mats, o = [], gap
    for r, c in shapes:
        mats.append((o, r, c))
        o += r * c + gap
    return mats, o + gap


@pytest.mark.parametrize("ns_dtype,pdt", [("bf16", "bf16"), ("fp32", "fp32"), ("bf16", "fp32")])
def test_muon_ragged_edge_shapes(gpu, ns_dtype, pdt):
    mats, n = _flat(EDGE_SHAPES)
    s = Setup(mats, n, pdt, pdt, ns_dtype, gpu, seed=3)
    check_muon_step(s, mhp(QUINTIC), tol_w=1e-2 if pdt == "bf16" else 1e-4)


# row starts on 4-element boundaries: the 4-wide momentum / apply paths,
# tall and wide, with rows off the 64-row tile grid
ALIGNED_SHAPES = [(36, 100), (100, 36), (130, 516), (516, 132), (4, 8), (8, 4), (64, 64)]


@pytest.mark.parametrize("ns_dtype,pdt", [("bf16", "bf16"), ("fp32", "fp32")])
def test_muon_vector_paths_aligned_ragged(gpu, ns_dtype, pdt):
    mats, n = _flat(ALIGNED_SHAPES, gap=4)
    assert all(o % 4 == 0 and c % 4 == 0 for o, r, c in mats)
    s = Setup(mats, n, pdt, pdt, ns_dtype, gpu, seed=4)
    check_muon_step(s, mhp(QUINTIC), tol_w=1e-2 if pdt == "bf16" else 1e-4)


# small matrices (short side padded to 32 at most 128, m_k * n_k <= 32768)
# run one NS iteration per launch in one workgroup; mixed with tiled ones
SMALL_SHAPES = [(128, 256), (256, 128), (96, 200), (200, 96), (17, 300), (1, 8), (32, 1000),
                (64, 64), (100, 320), (300, 520), (129, 200)]


@pytest.mark.parametrize("coef", [QUINTIC, CUBIC])
@pytest.mark.parametrize("pdt", ["bf16", "fp32"])
def test_small_matrix_kernel_is_bitwise_the_tiled_path(gpu, coef, pdt):
    mats, n = _flat(SMALL_SHAPES)
    fused = Setup(mats, n, pdt, pdt, "bf16", gpu, seed=8)
    tiled = Setup(mats, n, pdt, pdt, "bf16", gpu, seed=8, tiled_only=True)
    # (100, 320): m_k * n_k = 128 * 320 > 32768; (300, 520), (129, 200): m_k > 128
    assert fused.plan.info().small_mats == 8 and tiled.plan.info().small_mats == 0
    hp = mhp(coef)
    for _ in range(2):  # two steps: the second starts from a nonzero momentum
        fused.step(hp)
        tiled.step(hp)
    torch.cuda.synchronize()
    for a, b in ((fused.params, tiled.params), (fused.mom, tiled.mom), (fused.out, tiled.out)):
        assert torch.equal(a, b)


# diagonal tiles of the symmetric products split into upper blocks; with a
# short side padded to more than 8 tiles ((2304, 2400): 9) they run after
# the off-diagonal tiles; (64, 64) is on the fused small-matrix path
DIAG_SHAPES = [(2048, 2100), (2100, 2048), (300, 520), (520, 300), (1000, 700), (2304, 2400),
               (64, 64)]


@pytest.mark.parametrize("coef", [QUINTIC, CUBIC])
def test_split_diagonal_tiles_are_bitwise_whole_tiles(gpu, coef):
    mats, n = _flat(DIAG_SHAPES)
    split = Setup(mats, n, "bf16", "bf16", "bf16", gpu, seed=14)
    whole = Setup(mats, n, "bf16", "bf16", "bf16", gpu, seed=14, whole_tiles=True)
    assert split.plan.info().split_tile_mats == 6 and whole.plan.info().split_tile_mats == 0
    assert split.plan.info().small_mats == 1
    hp = mhp(coef)
    for _ in range(2):
        split.step(hp)
        whole.step(hp)
    torch.cuda.synchronize()
    for a, b in ((split.params, whole.params), (split.mom, whole.mom), (split.out, whole.out)):
        assert torch.equal(a, b)


def test_small_matrices_match_oracle(gpu):
    mats, n = _flat(SMALL_SHAPES[:8])
    s = Setup(mats, n, "bf16", "bf16", "bf16", gpu, seed=12)
    assert s.plan.info().small_mats == 8
    check_muon_step(s, mhp(QUINTIC), tol_w=1e-2)


@pytest.mark.parametrize("ns_dtype,pdt", [("bf16", "bf16"), ("fp32", "fp32")])
def test_grouped_equals_single_matrix_plans(gpu, ns_dtype, pdt):
    mats, n = _flat([(200, 700), (700, 200), (256, 256), (33, 99)])
    s = Setup(mats, n, pdt, pdt, ns_dtype, gpu, seed=5)
    P0, G0, M0 = s.params.clone(), s.grads.clone(), s.mom.clone()
    hp = mhp(QUINTIC)
    s.step(hp)
    grouped = s.out.clone()
    for k, m in enumerate(mats):
        s1 = Setup([m], n, pdt, pdt, ns_dtype, gpu, seed=5)
        s1.params.copy_(P0)
        s1.grads.copy_(G0)
        s1.mom.copy_(M0)
        s1.step(hp)
        o, r, c = m
        assert torch.equal(s1.out[o:o + r * c], grouped[o:o + r * c]), k


@pytest.mark.parametrize("ns_dtype,pdt", [("bf16", "bf16"), ("fp32", "fp32")])
def test_determinism_waves_and_stage_composition(gpu, ns_dtype, pdt):
    mats, n = _flat([(300, 520), (520, 300), (512, 512), (64, 1000), (1000, 64)])
    hp = mhp(QUINTIC)
    ref = Setup(mats, n, pdt, pdt, ns_dtype, gpu, seed=9)
    P0, G0, M0 = ref.params.clone(), ref.grads.clone(), ref.mom.clone()
    ref.step(hp)
    results = [(ref.params.clone(), ref.mom.clone(), ref.out.clone())]
    # same plan again, from the same state
    ref.params.copy_(P0)
    ref.mom.copy_(M0)
    ref.out.fill_(7.0)
    ref.step(hp)
    results.append((ref.params.clone(), ref.mom.clone(), ref.out.clone()))
    # capped workspace -> several waves
    one = M.muon_workspace_size(mats[:1], n, pdt, pdt, ns_dtype)
    capped = Setup(mats, n, pdt, pdt, ns_dtype, gpu, seed=9, cap=2 * one)
    assert capped.plan.info().n_waves > 1
    capped.params.copy_(P0)
    capped.mom.copy_(M0)
    capped.step(hp)
    results.append((capped.params.clone(), capped.mom.clone(), capped.out.clone()))
    # stage by stage, through the stage entry points
    st = Setup(mats, n, pdt, pdt, ns_dtype, gpu, seed=9)
    st.params.copy_(P0)
    st.mom.copy_(M0)
    M.muon_stage_momentum(st.plan, 0, G0, st.mom, st.ws, hp)
    for it in range(hp.ns_steps):
        for ph in (1, 2, 3):
            M.muon_stage_ns_phase(st.plan, 0, st.ws, hp, it, ph)
    M.muon_stage_apply(st.plan, 0, st.params, st.ws, hp, st.out)
    results.append((st.params.clone(), st.mom.clone(), st.out.clone()))
    for r in results[1:]:
        for a, b in zip(results[0], r):
            assert torch.equal(a, b)


def test_resume_is_bitwise(gpu):
    mats, n = _flat([(128, 384), (384, 128)])
    hp = mhp(CUBIC)
    a = Setup(mats, n, "bf16", "bf16", "bf16", gpu, seed=11)
    b = Setup(mats, n, "bf16", "bf16", "bf16", gpu, seed=11)
    g = torch.Generator(device=gpu)
    grads = []
    for k in range(4):
        g.manual_seed(100 + k)
        grads.append(torch.randn(n, generator=g, device=gpu).to(torch.bfloat16))
    for k in range(4):
        a.grads.copy_(grads[k])
        a.step(hp)
    for k in range(2):
        b.grads.copy_(grads[k])
        b.step(hp)
    saved = (b.params.cpu().clone(), b.mom.cpu().clone())
    b = Setup(mats, n, "bf16", "bf16", "bf16", gpu, seed=12)
    b.params.copy_(saved[0])
    b.mom.copy_(saved[1])
    for k in range(2, 4):
        b.grads.copy_(grads[k])
        b.step(hp)
    assert torch.equal(a.params, b.params) and torch.equal(a.mom, b.mom)


def test_stepwise_momentum_norm_and_iterates(gpu):
    for ns_dtype in ("fp32", "bf16"):
        mats, n = _flat([(96, 200), (200, 96)])
        s = Setup(mats, n, "fp32", "fp32", ns_dtype, gpu, seed=13)
        s.mom[:] = torch.randn(n, generator=_gen(gpu, 131), device=gpu) * 0.1
        hp = mhp(QUINTIC)
        P0, G0, M0 = s.snapshot()
        M.muon_stage_momentum(s.plan, 0, s.grads, s.mom, s.ws, hp)
        U = torch.zeros(n, device=gpu)
        norms = torch.zeros(len(mats), device=gpu)
        M.muon_stage_export_x(s.plan, 0, s.ws, 0, U)
        M.muon_stage_export_norms(s.plan, 0, s.ws, norms)
        torch.cuda.synchronize()
        tol_u = 2e-6 if ns_dtype == "fp32" else 4e-3
        Xs = []
        for i, (o, r, c) in enumerate(mats):
            sl = slice(o, o + r * c)
            Mr = O.ema_momentum(M0[sl], G0[sl], hp.momentum)
            Ur = O.nesterov_lookahead(Mr, G0[sl], hp.momentum, True)
            assert rel(np64(s.mom[sl]), Mr) <= 2e-6
            assert rel(np64(U[sl]), Ur) <= tol_u
            assert abs(np64(norms)[i] - np.linalg.norm(Ur)) <= 1e-6 * np.linalg.norm(Ur)
            Xs.append(O.frobenius_normalise(Ur.reshape(r, c), hp.eps))
        for it in range(hp.ns_steps):
            for ph in (1, 2, 3):
                M.muon_stage_ns_phase(s.plan, 0, s.ws, hp, it, ph)
            X = torch.zeros(n, device=gpu)
            M.muon_stage_export_x(s.plan, 0, s.ws, it + 1, X)
            torch.cuda.synchronize()
            for i, (o, r, c) in enumerate(mats):
                Xs[i] = O.newton_schulz(Xs[i], hp.ns_a, hp.ns_b, hp.ns_c, 1)
                assert rel(np64(X[o:o + r * c]).reshape(r, c), Xs[i]) <= TOL_O[ns_dtype], \
                    (ns_dtype, it, i)


@pytest.mark.parametrize("variant", ["ns0", "other_coefs", "no_nesterov", "mode1", "mode2",
                                     "zero_grad"])
def test_muon_hyperparameter_variants(gpu, variant):
    mats, n = _flat([(64, 320), (320, 64), (130, 130)])
    s = Setup(mats, n, "bf16", "bf16", "bf16", gpu, seed=17)
    hp = mhp(CUBIC)
    if variant == "ns0":
        hp.ns_steps = 0
    elif variant == "other_coefs":
        hp = mhp((2.0, -1.5, 0.5), steps=3)
    elif variant == "no_nesterov":
        hp.nesterov = False
        s.mom[:] = torch.randn(n, generator=_gen(gpu, 132), device=gpu) * 0.1
    elif variant == "mode1":
        hp.scale_mode = 1
    elif variant == "mode2":
        hp.scale_mode = 2
    elif variant == "zero_grad":
        for (o, r, c) in mats:
            s.grads[o:o + r * c] = 0
    check_muon_step(s, hp)
    if variant == "zero_grad":
        assert float(s.out[mats[0][0]:mats[0][0] + 64 * 320].abs().max()) == 0.0


def test_empty_plan_and_bad_workspace(gpu):
    p = M.muon_plan_create([], 0, "bf16", "bf16", "bf16")
    z = torch.zeros(16, dtype=torch.bfloat16, device=gpu)
    zm = torch.zeros(16, device=gpu)
    ws = torch.zeros(256, dtype=torch.uint8, device=gpu)
    M.muon_step(p, z, z, zm, ws, mhp())
    mats, n = _flat([(64, 64)])
    s = Setup(mats, n, "bf16", "bf16", "bf16", gpu)
    small = torch.zeros(s.plan.workspace_bytes - 256, dtype=torch.uint8, device=gpu)
    with pytest.raises(M.MuonError) as e:
        M.muon_step(s.plan, s.params, s.grads, s.mom, small, mhp())
    assert e.value.status == M.MUON_ERR_WORKSPACE_TOO_SMALL
    big = torch.zeros(s.plan.workspace_bytes + 512, dtype=torch.uint8, device=gpu)
    with pytest.raises(M.MuonError) as e:
        M.muon_step(s.plan, s.params, s.grads, s.mom, big[1:], mhp())
    assert e.value.status == M.MUON_ERR_INVALID_ARG
    with pytest.raises(M.MuonError):
        M.muon_step(s.plan, s.params, s.grads, s.mom, s.ws, mhp(steps=-1))


# ---------------------------------------------------------------- full-size workloads


def _workload_sampled(gpu, name, sample, hp, cap=0, first=None):
    wl = W.workload(name)
    if first is not None:  # the first `first` matrices of the workload, at full size
        wl.shapes = wl.shapes[:first]
    inp = W.make_muon_inputs(wl, gpu, step=1)
    plan = M.muon_plan_create(wl.mats(), wl.muon_numel(), wl.param_dtype, wl.grad_dtype,
                              "bf16", cap)
    ws = plan.alloc_workspace(gpu)
    out = torch.zeros(wl.muon_numel(), device=gpu)
    mats = wl.mats()
    before = {i: (np64(inp.params[o:o + r * c]), np64(inp.grads[o:o + r * c]),
                  np64(inp.momentum[o:o + r * c])) for i, (o, r, c) in
              ((i, mats[i]) for i in sample)}
    M.muon_step(plan, inp.params, inp.grads, inp.momentum, ws, hp, out)
    torch.cuda.synchronize()
    for i in sample:
        o, r, c = mats[i]
        Wn, Mn, On = O.muon_matrix_math(before[i][0].reshape(r, c), before[i][1].reshape(r, c),
                                        before[i][2].reshape(r, c), ohp(hp))
        sl = slice(o, o + r * c)
        assert rel(np64(out[sl]).reshape(r, c), On) <= 1e-2, (name, i, r, c)
        assert rel(np64(inp.momentum[sl]), O.fp32_round(Mn).ravel()) <= 2e-6, (name, i)
        assert rel(np64(inp.params[sl]), O.bf16_round(Wn).ravel()) <= 1e-2, (name, i)
    del ws, inp, out
    torch.cuda.empty_cache()


def test_dense_stack_full_size_sampled(gpu):
    # 16 layers x (4 x 2048^2, 2 x 2048x5632, 5632x2048), quintic, as timed
    _workload_sampled(gpu, "dense_d2048_l16", [0, 4, 6, 111], mhp(QUINTIC))


def test_moe_e64_full_size_sampled(gpu):
    _workload_sampled(gpu, "moe_e64_2048x1408", [0, 127, 150], mhp(QUINTIC))


def test_moe_e384_shapes_sampled(gpu):
    # 8 experts x (gate, up 7168x2048; down 2048x7168): the large expert
    # shapes of the 384-expert workload; matrices 0 (gate), 8 (up) and 16
    # (down, tall)
    wl = W.workload("moe_e384_7168x2048")
    shapes = wl.shapes[:8] + wl.shapes[384:392] + wl.shapes[768:776]
    assert shapes[0] == (7168, 2048) and shapes[16] == (2048, 7168)
    wl.shapes = shapes
    inp = W.make_muon_inputs(wl, gpu, step=1)
    hp = mhp(QUINTIC)
    plan = M.muon_plan_create(wl.mats(), wl.muon_numel(), "bf16", "bf16", "bf16")
    ws = plan.alloc_workspace(gpu)
    out = torch.zeros(wl.muon_numel(), device=gpu)
    mats = wl.mats()
    before = {i: tuple(np64(t[o:o + r * c]) for t in (inp.params, inp.grads, inp.momentum))
              for i, (o, r, c) in ((i, mats[i]) for i in (0, 16))}
    M.muon_step(plan, inp.params, inp.grads, inp.momentum, ws, hp, out)
    torch.cuda.synchronize()
    for i in (0, 16):
        o, r, c = mats[i]
        Wn, Mn, On = O.muon_matrix_math(*(x.reshape(r, c) for x in before[i]), ohp(hp))
        assert rel(np64(out[o:o + r * c]).reshape(r, c), On) <= 1e-2, i
        assert rel(np64(inp.momentum[o:o + r * c]), O.fp32_round(Mn).ravel()) <= 2e-6


def test_ragged_shapes_full_size_sampled(gpu):
    # the first 40 shapes of the seeded ragged draw (square / tall / wide,
    # every tenth off the 64 grid), oracle on four of them including two
    # off-grid matrices
    wl = W.workload("ragged_500")
    shapes = wl.shapes[:40]
    small = sorted(range(40), key=lambda i: min(shapes[i]))
    sample = sorted(set([i for i in small if i % 10 == 0][:2] + small[:2]))
    _workload_sampled(gpu, "ragged_500", sample, mhp(QUINTIC), first=40)


@pytest.mark.parametrize("g_std,eps", [(1e14, 1e-7), (1e-25, 1e-7), (1e18, 1e-7), (1e-22, 0.0)])
def test_extreme_gradient_scales_normalise_like_the_oracle(gpu, g_std, eps):
    # ||U||_F outside [2^-40, 2^40]: the norm kernel scales U by a power of
    # two (folded into inv) before the first products, which otherwise
    # accumulate U U^T unnormalised in fp32.  |u| ~ 1e17: U U^T and inv^2
    # would leave the fp32 range; |u| ~ 1e-23 with eps = 0: inv^2 would
    # overflow and u^2 underflow; |u| ~ 1e-26 with eps = 1e-7: ||U||_F sits
    # far below eps.  Tiled and fused small-matrix paths, both NS dtypes.
    mats, n = _flat([(300, 520), (520, 300), (96, 200), (64, 64)])
    for nsd, pdt in (("bf16", "bf16"), ("fp32", "fp32")):
        s = Setup(mats, n, pdt, pdt, nsd, gpu, seed=17, w_std=0.02, g_std=g_std)
        worst = check_muon_step(s, mhp(QUINTIC, eps=eps))
        assert np.isfinite(np64(s.out)).all() and np.isfinite(np64(s.params)).all()
        assert worst["O"] <= TOL_O[nsd]
        norms = torch.zeros(len(mats), device=gpu)
        M.muon_stage_export_norms(s.plan, 0, s.ws, norms)
        torch.cuda.synchronize()
        assert np.isfinite(np64(norms)).all() and (np64(norms) > 0).all()


def test_span_path_matches_the_scalar_path(gpu):
    # Matrices at odd offsets or widths in an aligned buffer take the apply
    # kernel's span path (aligned 4-element groups of each tile row of W);
    # the same matrices in buffers shifted by one element (no 4-element
    # alignment anywhere) take its one-element path.  Both compute the same
    # expression per element, and the momentum and NS kernels take the same
    # paths in both layouts, so W, M and O agree bitwise.
    shapes = [(37, 129), (129, 37), (300, 517), (517, 300), (64, 65), (1000, 7)]
    mats, n = _flat(shapes, gap=5)
    hp = mhp(QUINTIC)
    res = []
    for shift in (0, 1):
        g = torch.Generator(device=gpu)
        g.manual_seed(41)
        P = torch.zeros(n + 8, dtype=torch.bfloat16, device=gpu)
        G = torch.zeros(n + 8, dtype=torch.bfloat16, device=gpu)
        Mo = torch.zeros(n + 8, device=gpu)
        out = torch.zeros(n + 8, device=gpu)
        vals = [(torch.randn(r * c, generator=g, device=gpu) * 0.02,
                 torch.randn(r * c, generator=g, device=gpu) * 0.02,
                 torch.randn(r * c, generator=g, device=gpu) * 1e-3) for (o, r, c) in mats]
        for (o, r, c), (w, gr, m) in zip(mats, vals):
            P[shift + o:shift + o + r * c] = w.to(torch.bfloat16)
            G[shift + o:shift + o + r * c] = gr.to(torch.bfloat16)
            Mo[shift + o:shift + o + r * c] = m
        plan = M.muon_plan_create(mats, n, "bf16", "bf16", "bf16")
        ws = plan.alloc_workspace(gpu)
        for with_out in (True, False):
            M.muon_step(plan, P[shift:shift + n], G[shift:shift + n], Mo[shift:shift + n], ws, hp,
                        out[shift:shift + n] if with_out else None)
        torch.cuda.synchronize()
        res.append((P[shift:shift + n].clone(), Mo[shift:shift + n].clone(),
                    out[shift:shift + n].clone()))
    (P0, M0, O0), (P1, M1, O1) = res
    assert torch.equal(M0, M1) and torch.equal(O0, O1)
    assert torch.equal(P0.view(torch.int16), P1.view(torch.int16))
