"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these retypes the oracle's formula: each compares it with a closed
form, a spectral-calculus identity computed through an SVD, an invariant,
a library routine (torch's bf16 cast) or a value the pages print
(tests/golden/, each file citing its source).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import muon_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- rounding


def test_bf16_round_hand_cases():
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing at 1.0
    cases = {
        one: one,
        one + ulp / 2: one,               # exact tie -> even (1.0)
        one + 3 * ulp / 2: one + 2 * ulp,  # exact tie -> even (1 + 2 ulp)
        one + ulp / 2 + 2.0 ** -20: one + ulp,  # just above the tie
        -(one + ulp / 2): -one,
        0.0: 0.0,
    }
    for x, want in cases.items():
        assert O.bf16_round(np.array([x]))[0] == want, x
    assert np.isnan(O.bf16_round(np.array([np.nan]))[0])
    assert np.isinf(O.bf16_round(np.array([np.inf]))[0])


def test_bf16_round_matches_torch_cast():
    x = np.concatenate([rng(0).standard_normal(20000) * s for s in (1e-30, 1e-4, 1.0, 1e30)])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)


# ---------------------------------------------------------------- AdamW


def test_adamw_first_step_closed_form():
    # From a zero state, t = 1: m_hat = g, v_hat = g^2, so the step is
    # theta1 = (1 - lr*wd) theta0 - lr * g / (|g| + eps).  A large eps and
    # large lr*wd make eps placement and the decay term visible.
    hp = O.AdamWHP(lr=0.5, beta1=0.9, beta2=0.95, eps=1e-2, weight_decay=0.3)
    r = rng(1)
    th0 = r.standard_normal(1000)
    g = r.standard_normal(1000) * np.logspace(-4, 1, 1000)
    th1, m1, v1 = O.adamw_math(th0, g, np.zeros(1000), np.zeros(1000), hp, 1)
    want = (1 - hp.lr * hp.weight_decay) * th0 - hp.lr * g / (np.abs(g) + hp.eps)
    np.testing.assert_allclose(th1, want, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(m1, (1 - hp.beta1) * g, rtol=1e-15)
    np.testing.assert_allclose(v1, (1 - hp.beta2) * g * g, rtol=1e-15)


@pytest.mark.parametrize("beta1,beta2", [(0.9, 0.95), (0.9, 0.999), (0.5, 0.3)])
def test_adamw_constant_gradient_closed_form(beta1, beta2):
    # Constant g from zero state: bias correction makes m_hat = g and
    # v_hat = g^2 for every t, so each step is the same: with d = 1 - lr*wd,
    # theta_T = d^T theta0 - lr*g/(|g|+eps) * sum_{s<T} d^s.
    hp = O.AdamWHP(lr=0.1, beta1=beta1, beta2=beta2, eps=1e-3, weight_decay=0.2)
    r = rng(2)
    th = th0 = r.standard_normal(64)
    g = r.standard_normal(64)
    m = np.zeros(64)
    v = np.zeros(64)
    T = 10
    for t in range(1, T + 1):
        th, m, v = O.adamw_math(th, g, m, v, hp, t)
    d = 1 - hp.lr * hp.weight_decay
    want = d ** T * th0 - hp.lr * g / (np.abs(g) + hp.eps) * sum(d ** s for s in range(T))
    np.testing.assert_allclose(th, want, rtol=1e-12)
    np.testing.assert_allclose(m, (1 - beta1 ** T) * g, rtol=1e-13)
    np.testing.assert_allclose(v, (1 - beta2 ** T) * g * g, rtol=1e-13)


def test_adamw_zero_betas_reduce_to_sign_like_step():
    # beta1 = beta2 = 0: m_hat = g_t and v_hat = g_t^2 regardless of history.
    hp = O.AdamWHP(lr=0.3, beta1=0.0, beta2=0.0, eps=0.05, weight_decay=0.0)
    r = rng(3)
    th = r.standard_normal(32)
    m = r.standard_normal(32)
    v = np.abs(r.standard_normal(32))
    for t in range(1, 5):
        g = r.standard_normal(32)
        th_new, m, v = O.adamw_math(th, g, m, v, hp, t)
        np.testing.assert_allclose(th_new, th - hp.lr * g / (np.abs(g) + hp.eps), rtol=1e-14)
        th = th_new


def test_adamw_gradient_scale_invariance_without_eps():
    hp = O.AdamWHP(lr=0.1, beta1=0.9, beta2=0.95, eps=0.0, weight_decay=0.1)
    r = rng(4)
    th = r.standard_normal(50)
    gs = [r.standard_normal(50) for _ in range(4)]
    a = (th, np.zeros(50), np.zeros(50))
    b = (th, np.zeros(50), np.zeros(50))
    for t, g in enumerate(gs, 1):
        a = O.adamw_math(a[0], g, a[1], a[2], hp, t)
        b = O.adamw_math(b[0], 1e3 * g, b[1], b[2], hp, t)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12)


def test_adamw_rejects_step_zero():
    with pytest.raises(ValueError):
        O.adamw_math(np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1), O.AdamWHP(), 0)


def test_adamw_stored_param_is_cast_of_fp32_master():
    hp = O.AdamWHP()
    r = rng(5)
    master = O.fp32_round(r.standard_normal(4096) * 0.02)
    param = O.bf16_round(master)
    g = O.bf16_round(r.standard_normal(4096) * 0.02)
    p1, m1, a1, b1 = O.adamw_step_stored(param, master, g, np.zeros(4096), np.zeros(4096),
                                         hp, 1, "bf16")
    ref = torch.from_numpy(m1.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(p1, ref)
    assert m1.dtype == np.float64 and np.all(O.fp32_round(m1) == m1)


def test_adam_hparam_defaults_match_page():
    gold = _golden("opt_tutorial_adam_hparams.json")
    hp = O.AdamWHP()
    assert hp.beta1 == gold["beta1_default"]
    assert hp.beta2 in gold["beta2_llm"]
    assert hp.eps == gold["eps_default"]


# ---------------------------------------------------------------- momentum


@pytest.mark.parametrize("mu", [0.9, 0.95])
def test_momentum_constant_gradient_closed_form(mu):
    # EMA from zero with constant g: M_t = (1 - mu^t) g; the Nesterov
    # look-ahead is mu*M_t + (1-mu) g = (1 - mu^(t+1)) g.
    g = rng(6).standard_normal((5, 7))
    M = np.zeros_like(g)
    for t in range(1, 12):
        M = O.ema_momentum(M, g, mu)
        np.testing.assert_allclose(M, (1 - mu ** t) * g, rtol=1e-13)
        np.testing.assert_allclose(O.nesterov_lookahead(M, g, mu, True),
                                   (1 - mu ** (t + 1)) * g, rtol=1e-13)
        np.testing.assert_array_equal(O.nesterov_lookahead(M, g, mu, False), M)


# ---------------------------------------------------------------- Newton-Schulz


def _scalar_poly_iter(s, a, b, c, steps):
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def _spectral_reference(X0, a, b, c, steps):
    U, s, Vt = np.linalg.svd(X0, full_matrices=False)
    return (U * _scalar_poly_iter(s, a, b, c, steps)) @ Vt


COEFFS = [(1.5, -0.5, 0.0), (15 / 8, -5 / 4, 3 / 8), (2.0, -1.5, 0.5)]


@pytest.mark.parametrize("shape", [(4, 7), (16, 16), (33, 17), (128, 256), (7, 4), (1, 9), (9, 1)])
@pytest.mark.parametrize("coef", COEFFS)
@pytest.mark.parametrize("steps", [1, 2, 5])
def test_ns_equals_scalar_polynomial_on_singular_values(shape, coef, steps):
    # The NS step is an odd matrix polynomial, so it acts on each singular
    # value separately: O = U diag(p^k(sigma)) V^T.
    G = rng(hash((shape, steps)) % 2 ** 32).standard_normal(shape)
    X0 = O.frobenius_normalise(G, 1e-7)
    got = O.newton_schulz(X0, *coef, steps)
    want = _spectral_reference(X0, *coef, steps)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13 * max(1.0, np.abs(want).max()))


def test_ns_cubic_is_the_printed_iteration():
    gold = _golden("opt_tutorial_ns_cubic.json")
    X = O.frobenius_normalise(rng(7).standard_normal((6, 10)), 1e-7)
    got = O.ns_iteration(X, gold["a"], gold["b"], gold["c"])
    np.testing.assert_allclose(got, (3 * X - X @ X.T @ X) / 2, rtol=1e-14, atol=1e-16)
    # p(1) = a + b + c = 1: the printed iteration fixes singular value 1
    assert gold["a"] + gold["b"] + gold["c"] == gold["fixed_point_sigma"]


def test_ns_tall_equals_right_multiplied_form():
    # For tall X the oracle iterates X^T; compare with the untransposed
    # form X <- a X + X (b S + c S S), S = X^T X (same polynomial).
    X = O.frobenius_normalise(rng(8).standard_normal((40, 12)), 1e-7)
    a, b, c = COEFFS[1]
    Y = X.copy()
    for _ in range(5):
        S = Y.T @ Y
        Y = a * Y + Y @ (b * S + c * S @ S)
    np.testing.assert_allclose(O.newton_schulz(X, a, b, c, 5), Y, atol=1e-14)
    np.testing.assert_allclose(O.newton_schulz(X.T, a, b, c, 5), Y.T, atol=1e-14)


def test_ns_square_nonsymmetric_uses_x_xt():
    # X X^T X differs from X^T X X on a non-normal square matrix; the SVD pin
    # above fixes the operand order; this shows the two are distinguishable.
    X = O.frobenius_normalise(rng(9).standard_normal((8, 8)), 1e-7)
    a, b, c = COEFFS[0]
    wrong = a * X + b * (X.T @ X) @ X
    assert np.abs(O.ns_iteration(X, a, b, c) - wrong).max() > 1e-3


@pytest.mark.parametrize("coef", COEFFS[:2])
def test_ns_clips_spectral_norm(coef):
    # The polynomials map [0, 1] into [0, 1]: sigma_max(O) <= 1 whenever
    # sigma_max(X0) <= ||X0||_F <= 1 (Zhihu answer on K2, section 3.2: NS
    # clips the largest singular value; section 4: ||.||_2 <= ||.||_F).
    for seed in range(5):
        X0 = O.frobenius_normalise(rng(10 + seed).standard_normal((30, 50)), 1e-7)
        assert np.linalg.norm(X0, 2) <= 1.0
        Ok = O.newton_schulz(X0, *coef, 5)
        assert np.linalg.norm(Ok, 2) <= 1.0 + 1e-12


def test_ns_converges_to_orthogonal_with_enough_steps():
    # The iteration pushes every singular value toward 1 (tutorial 4.2);
    # 5 cubic steps are not enough from a Gaussian start, 15 are.
    X0 = O.frobenius_normalise(rng(11).standard_normal((128, 256)), 1e-7)
    I = np.eye(128)
    O15 = O.newton_schulz(X0, 1.5, -0.5, 0.0, 15)
    assert np.linalg.norm(O15 @ O15.T - I, 2) < 1e-8
    O5 = O.newton_schulz(X0, 1.5, -0.5, 0.0, 5)
    assert np.linalg.norm(O5 @ O5.T - I, 2) > 0.5


def test_ns_zero_and_diagonal_and_rank1():
    np.testing.assert_array_equal(O.newton_schulz(np.zeros((5, 9)), 1.5, -0.5, 0, 5), 0)
    s = np.array([0.9, 0.5, 0.1, 0.0])
    D = np.zeros((4, 6))
    D[np.arange(4), np.arange(4)] = s
    want = np.zeros((4, 6))
    want[np.arange(4), np.arange(4)] = _scalar_poly_iter(s, *COEFFS[1], 5)
    np.testing.assert_allclose(O.newton_schulz(D, *COEFFS[1], 5), want, atol=1e-15)
    u, v = rng(12).standard_normal(7), rng(13).standard_normal(11)
    G = np.outer(u, v)
    eps = 1e-7
    X0 = O.frobenius_normalise(G, eps)
    sig = np.linalg.norm(G) / (np.linalg.norm(G) + eps)
    want = _scalar_poly_iter(sig, *COEFFS[0], 5) * G / np.linalg.norm(G)
    np.testing.assert_allclose(O.newton_schulz(X0, *COEFFS[0], 5), want, atol=1e-14)


def test_normalise_scale_invariance():
    U = rng(14).standard_normal((9, 13))
    np.testing.assert_allclose(O.frobenius_normalise(1e4 * U, 1e-7),
                               O.frobenius_normalise(U, 1e-7), rtol=1e-7)
    assert abs(np.linalg.norm(O.frobenius_normalise(U, 0.0)) - 1.0) < 1e-14


# ---------------------------------------------------------------- scale and apply


def _orthonormal_rows(m, n, seed):
    Q, _ = np.linalg.qr(rng(seed).standard_normal((n, m)))
    return Q.T  # m x n with orthonormal rows


def test_scale_mode0_matches_rms_target():
    # Zhihu answer on K2, section 3.1: match the update RMS to AdamW's
    # (0.2-0.4).  For O with orthonormal rows (m <= n) ||O||_F^2 = m.
    for (r, c) in [(64, 256), (256, 64), (100, 100)]:
        Q = _orthonormal_rows(min(r, c), max(r, c), r + c)
        Om = Q if r <= c else Q.T
        s = O.update_scale(r, c, 0, 0.2)
        rms = np.sqrt(np.mean((s * Om) ** 2))
        assert abs(rms - 0.2) < 1e-12


def test_scale_modes_1_and_2():
    assert O.update_scale(2048, 5632, 1, 0.2) == 1.0
    assert abs(O.update_scale(5632, 2048, 1, 0.2) - math.sqrt(5632 / 2048)) < 1e-15
    assert O.update_scale(7, 3, 2, 0.2) == 1.0


@pytest.mark.parametrize("nesterov", [True, False])
@pytest.mark.parametrize("shape", [(16, 48), (48, 16)])
def test_muon_matrix_step_closed_form_on_orthonormal_gradient(nesterov, shape):
    # Zero momentum and G with orthonormal rows (or columns): U = k*G with
    # k = (1-mu^2) (Nesterov) or (1-mu); every singular value of X0 is
    # sigma0 = k/(k*sqrt(m) + eps), so O = p^steps(sigma0)/sigma0 * X0 and
    # W1 = (1 - lr*wd) W0 - lr*s*O.
    r, c = shape
    m = min(r, c)
    Q = _orthonormal_rows(m, max(r, c), 20)
    G = Q if r <= c else Q.T
    hp = O.MuonHP(lr=0.05, weight_decay=0.3, momentum=0.9, nesterov=nesterov,
                  ns_a=15 / 8, ns_b=-5 / 4, ns_c=3 / 8, ns_steps=5, eps=1e-3)
    W0 = rng(21).standard_normal(shape)
    W1, M1, Oout = O.muon_matrix_math(W0, G, np.zeros(shape), hp)
    k = (1 - hp.momentum ** 2) if nesterov else (1 - hp.momentum)
    sigma0 = k / (k * math.sqrt(m) + hp.eps)
    p = _scalar_poly_iter(sigma0, hp.ns_a, hp.ns_b, hp.ns_c, hp.ns_steps)
    O_want = p * G
    np.testing.assert_allclose(Oout, O_want, atol=1e-13)
    s = 0.2 * math.sqrt(max(r, c))
    np.testing.assert_allclose(W1, (1 - 0.05 * 0.3) * W0 - 0.05 * s * O_want, atol=1e-13)
    np.testing.assert_allclose(M1, (1 - hp.momentum) * G, atol=1e-15)


def test_muon_zero_gradient_is_pure_decay():
    hp = O.MuonHP()
    W0 = rng(22).standard_normal((8, 8))
    W1, M1, Oo = O.muon_matrix_math(W0, np.zeros((8, 8)), np.zeros((8, 8)), hp)
    np.testing.assert_array_equal(Oo, 0)
    np.testing.assert_allclose(W1, (1 - hp.lr * hp.weight_decay) * W0, rtol=1e-15)


def test_muon_flat_buffer_matches_per_matrix_and_keeps_gaps():
    # Flat concatenation with per-matrix offsets (Zhihu answer on K2, 2.2).
    shapes = [(5, 9), (12, 4), (3, 3)]
    mats, off = [], 3
    for r, c in shapes:
        mats.append((off, r, c))
        off += r * c + 2               # gaps of two untouched elements
    n = off + 5
    r = rng(23)
    P = O.bf16_round(r.standard_normal(n))
    Gf = O.bf16_round(r.standard_normal(n))
    Mf = O.fp32_round(r.standard_normal(n) * 0.1)
    hp = O.MuonHP()
    P1, M1, outs = O.muon_step_flat(P, Gf, Mf, mats, hp, "bf16")
    covered = np.zeros(n, bool)
    for i, (o, rr, cc) in enumerate(mats):
        sl = slice(o, o + rr * cc)
        covered[sl] = True
        W1, Mn, Oo = O.muon_matrix_math(P[sl].reshape(rr, cc), Gf[sl].reshape(rr, cc),
                                        Mf[sl].reshape(rr, cc), hp)
        np.testing.assert_array_equal(P1[sl], O.bf16_round(W1).ravel())
        np.testing.assert_array_equal(M1[sl], O.fp32_round(Mn).ravel())
        np.testing.assert_array_equal(outs[i], Oo)
    np.testing.assert_array_equal(P1[~covered], P[~covered])
    np.testing.assert_array_equal(M1[~covered], Mf[~covered])
    _, _, part = O.muon_step_flat(P, Gf, Mf, mats, hp, "bf16", only=[1])
    assert list(part) == [1]


# ---------------------------------------------------------------- accounting


def test_ns_flop_count_brute_force():
    # count multiply-adds of one triangle of X X^T, one triangle of A A and
    # the full B X by enumeration on a tiny case
    m, n = 5, 7
    syrk = sum(2 * n for i in range(m) for j in range(i, m))
    sq = sum(2 * m for i in range(m) for j in range(i, m))
    bx = 2 * m * m * n
    assert O.ns_flops(m, n, 1, 0.0) == syrk + bx
    assert O.ns_flops(n, m, 3, 0.1) == 3 * (syrk + sq + bx)


def test_state_bytes_match_memory_table():
    from muon_newton_schulz_amd.workloads import optimizer_state_bytes
    gold = _golden("opt_tutorial_memory_table.json")
    n = int(gold["n_params"])
    for k, gb in gold["extra_state_GB"].items():
        assert optimizer_state_bytes(n, k) == gb * 1e9, k
    assert n * 4 == gold["fp32_master_GB"] * 1e9
    assert n * 2 == gold["fp16_weights_GB"] * 1e9
    assert optimizer_state_bytes(n, "adamw") + n * 4 == gold["adamw_related_total_GB"] * 1e9
    assert O.muon_state_bytes_per_param() * n == gold["muon_vs_adam_state_ratio"] * optimizer_state_bytes(n, "adamw")
