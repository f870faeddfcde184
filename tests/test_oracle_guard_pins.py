"""Pins of oracle/guard_oracle.py (gradient clipping, the non-finite guard,
optimizer-state statistics) and of the clip factor's use in the Muon and
AdamW oracles, against closed forms and properties of the method."""

import math

import numpy as np
import pytest

from oracle import guard_oracle as G
from oracle import muon_oracle as O


def test_global_norm_of_constant_buffers():
    # 16 elements of 0.25 split over two buffers: sqrt(16 * 0.0625) = 1
    bufs = [np.full(5, 0.25, np.float32), np.full(11, -0.25, np.float64)]
    assert G.global_grad_norm(bufs) == 1.0


def test_global_norm_three_four_five():
    assert G.global_grad_norm([np.array([3.0]), np.array([4.0])]) == 5.0
    assert G.global_grad_norm([np.array([3.0, 0.0, 0.0]), np.zeros(0), np.array([0.0, -4.0])]) == 5.0
    assert G.global_grad_norm([np.zeros(7)]) == 0.0
    assert G.global_grad_norm([]) == 0.0


def test_global_norm_non_finite():
    assert math.isnan(G.global_grad_norm([np.array([1.0, np.nan])]))
    assert G.global_grad_norm([np.array([1.0]), np.array([-np.inf])]) == math.inf
    # fp32 extremes do not overflow the fp64 sum of squares
    big = np.full(1000, np.finfo(np.float32).max, np.float32)
    n = G.global_grad_norm([big])
    assert math.isfinite(n)
    assert n == pytest.approx(float(np.finfo(np.float32).max) * math.sqrt(1000), rel=1e-12)


def test_guard_skip():
    assert G.guard_skip(math.nan) and G.guard_skip(math.inf)
    assert not G.guard_skip(0.0) and not G.guard_skip(1e300)


def test_clip_factor_cases():
    assert G.clip_factor(5.0, 1.0) == 1.0 / (5.0 + 1e-6)
    assert G.clip_factor(0.5, 1.0) == 1.0          # within the threshold: unchanged
    assert G.clip_factor(1.0 - 1e-6, 1.0) == 1.0   # exactly at the threshold after eps
    assert G.clip_factor(5.0, 0.0) == 1.0          # clipping disabled
    assert G.clip_factor(5.0, -2.0) == 1.0
    assert G.clip_factor(math.nan, 1.0) == 1.0     # the step is skipped anyway
    assert G.clip_factor(4.0, 2.0, eps=0.0) == 0.5
    # the clipped norm is max_norm (up to eps)
    g = np.arange(1.0, 10.0)
    n = G.global_grad_norm([g])
    f = G.clip_factor(n, 2.0)
    assert G.global_grad_norm([f * g]) == pytest.approx(2.0, rel=1e-6)


def test_clipped_first_muon_step_closed_forms():
    rng = np.random.default_rng(0)
    W = rng.standard_normal((6, 9))
    Gm = rng.standard_normal((6, 9))
    M0 = np.zeros((6, 9))
    hp = O.MuonHP()
    f = 0.3
    W1, M1, O1 = O.muon_matrix_math(W, Gm, M0, hp, grad_scale=f)
    W0, M0b, O0 = O.muon_matrix_math(W, Gm, M0, hp)
    # EMA from zero: M_1 = (1 - mu) * f * G
    np.testing.assert_allclose(M1, (1 - hp.momentum) * f * Gm, rtol=1e-15, atol=0)
    # the Frobenius normalisation removes the gradient scale (up to eps)
    np.testing.assert_allclose(O1, O0, rtol=0, atol=1e-5)
    assert not np.allclose(M1, M0b)


def test_clipped_first_adamw_step_closed_form():
    # t = 1 from zero state: m_hat = f g, v_hat = (f g)^2, so
    # theta_1 = theta_0 - lr * f g / (|f g| + eps) - lr * wd * theta_0
    hp = O.AdamWHP(lr=0.01, beta1=0.9, beta2=0.95, eps=1e-3, weight_decay=0.1)
    th = np.array([1.0, -2.0, 0.5, 0.0])
    g = np.array([0.004, -0.5, 2.0, 1e-4])
    f = 0.25
    th1, m1, v1 = O.adamw_math(th, g, np.zeros(4), np.zeros(4), hp, 1, grad_scale=f)
    fg = f * g
    want = th - hp.lr * fg / (np.abs(fg) + hp.eps) - hp.lr * hp.weight_decay * th
    np.testing.assert_allclose(th1, want, rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(m1, (1 - hp.beta1) * fg, rtol=1e-15)
    np.testing.assert_allclose(v1, (1 - hp.beta2) * fg * fg, rtol=1e-15)


def test_flat_wrappers_pass_the_scale():
    rng = np.random.default_rng(1)
    mats = [(0, 4, 5), (20, 3, 3)]
    p = rng.standard_normal(29)
    g = rng.standard_normal(29)
    m = rng.standard_normal(29)
    hp = O.MuonHP()
    _, mom_s, _ = O.muon_step_flat(p, g, m, mats, hp, "fp32", grad_scale=0.5)
    _, mom_1, _ = O.muon_step_flat(p, g, m, mats, hp, "fp32")
    # momentum moves by (1 - mu) * (f - 1) * g between the two
    np.testing.assert_allclose(mom_s - mom_1, (1 - hp.momentum) * (0.5 - 1.0) * g,
                               rtol=1e-6, atol=3e-7)
    ahp = O.AdamWHP()
    _, _, ms, _ = O.adamw_step_stored(p, None, g, m, np.abs(m), ahp, 3, "fp32", grad_scale=0.5)
    _, _, m1, _ = O.adamw_step_stored(p, None, g, m, np.abs(m), ahp, 3, "fp32")
    np.testing.assert_allclose(ms - m1, (1 - ahp.beta1) * (0.5 - 1.0) * g, rtol=1e-6, atol=3e-7)


def test_state_stats_arithmetic_sequence():
    a, d, n = -3.5, 0.25, 101
    x = a + d * np.arange(n)
    np.random.default_rng(2).shuffle(x)
    s = G.state_stats(x.astype(np.float32))
    assert s["count"] == n and s["nonfinite"] == 0
    assert s["mean"] == pytest.approx(a + d * (n - 1) / 2, rel=1e-14)
    # population variance of an arithmetic sequence: d^2 (n^2 - 1) / 12
    assert s["var"] == pytest.approx(d * d * (n * n - 1) / 12, rel=1e-13)
    assert s["min"] == a and s["max"] == a + d * (n - 1)
    assert s["absmax"] == max(abs(a), abs(a + d * (n - 1)))


def test_state_stats_skip_non_finite():
    x = np.linspace(1.0, 2.0, 9)
    y = np.concatenate([x[:3], [np.nan], x[3:6], [np.inf, -np.inf], x[6:]])
    sx, sy = G.state_stats(x), G.state_stats(y)
    assert sy["nonfinite"] == 3 and sy["count"] == 9
    for k in ("mean", "var", "min", "max", "absmax"):
        assert sy[k] == sx[k]
    z = G.state_stats(np.array([np.nan, np.inf]))
    assert z == {"count": 0, "nonfinite": 2, "mean": 0.0, "var": 0.0, "min": 0.0,
                 "max": 0.0, "absmax": 0.0}
    e = G.state_stats(np.zeros(0))
    assert e["count"] == 0 and e["nonfinite"] == 0


def test_state_stats_constant_and_sign():
    s = G.state_stats(np.full(1000, -7.0))
    assert s["mean"] == -7.0 and s["var"] == 0.0 and s["absmax"] == 7.0
    assert s["min"] == -7.0 and s["max"] == -7.0
