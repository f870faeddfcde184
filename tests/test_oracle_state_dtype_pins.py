"""Pins of the oracle's compressed AdamW states (reading R13: m in fp32 or
bf16, v in fp32, bf16 or fp16): the IEEE binary16 rounding against values
fixed by the format's definition, and the stored states of the first step
against closed forms."""

import math

import numpy as np
import pytest

from oracle import muon_oracle as O


def test_fp16_rounding_fixed_points():
    x = [1.0, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 65504.0, 65519.99, 65520.0, 2 ** -24, 2 ** -25,
         3 * 2 ** -26, 2 ** -14, 1 / 3, -2.5]
    want = [1.0,
            1.0,                 # halfway between 1 and 1 + 2^-10: ties to even
            1 + 2 ** -9,         # halfway between 1 + 2^-10 and 1 + 2^-9: ties to even (up)
            65504.0,             # largest finite
            65504.0,             # below the rounding boundary 65520
            math.inf,            # at the boundary: rounds to infinity
            2 ** -24,            # smallest subnormal
            0.0,                 # halfway between 0 and 2^-24: ties to even (0)
            2 ** -24,            # 0.75 * 2^-24 rounds up
            2 ** -14,            # smallest normal
            0.333251953125,      # 1/3 to 10 fraction bits (0x3555)
            -2.5]
    got = O.fp16_round(x)
    assert list(got) == want
    assert math.isnan(O.fp16_round([math.nan])[0])
    assert O.round_to([1 + 2 ** -11], "fp16")[0] == 1.0


def test_fp16_rounds_the_fp32_value():
    # The stored state is the fp16 rounding of the fp32 value the step
    # computes, not of the exact one.  1 + 2^-11 + 2^-30 is above the
    # midpoint between 1 and 1 + 2^-10, so it would round up directly; in
    # fp32 (23 fraction bits) it is the midpoint itself, which ties to 1.
    x = 1 + 2 ** -11 + 2 ** -30
    assert float(np.float16(x)) == 1 + 2 ** -10      # direct rounding, for contrast
    assert O.fp16_round([x])[0] == 1.0
    # the same for bf16 (8 significant bits): 1 + 2^-8 is the midpoint
    y = 1 + 2 ** -8 + 2 ** -30
    assert O.bf16_round([y])[0] == 1.0


def test_first_step_states_in_16_bit():
    # t = 1 from zero: m1 = (1 - b1) g, v1 = (1 - b2) g^2, stored rounded
    hp = O.AdamWHP(lr=0.01, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)
    g = np.array([2.0, -0.5, 3.0, 1e-4])
    th0 = np.zeros(4)
    p, _, m, v = O.adamw_step_stored(th0, None, g, np.zeros(4), np.zeros(4), hp, 1, "fp32",
                                     m_dtype="bf16", v_dtype="fp16")
    # 0.05 * 4 = 0.2 -> fp16 0x3266 = 0.199951171875
    assert v[0] == 0.199951171875
    # 0.05 * 0.25 = 0.0125 -> fp16 0x2266 = 0.0124969482421875
    assert v[1] == 0.0124969482421875
    # 0.05 * 9 = 0.45 -> fp16 0x3733 = 0.449951171875
    assert v[2] == 0.449951171875
    # 0.05 * 1e-8 = 5e-10 is below half the smallest subnormal: stored as 0
    assert v[3] == 0.0
    # m in bf16: 0.1 * 2 = 0.2 -> bf16 0x3e4d = 0.2001953125; -0.05 -> 0xbd4d
    assert m[0] == 0.2001953125
    assert m[1] == -0.050048828125
    # the update of this step used the unrounded states: theta1 = -lr g / (|g| + eps)
    np.testing.assert_allclose(p, -0.01 * g / (np.abs(g) + 1e-8), rtol=1e-6)


def test_underflowed_v_makes_the_next_step_large():
    # the hazard of fp16 v: v stored as 0 after step 1; at step 2 with g = 0,
    # m_hat / (sqrt(v_hat) + eps) = m_hat / eps
    hp = O.AdamWHP(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)
    g1 = np.array([1e-4])
    p1, _, m1, v1 = O.adamw_step_stored(np.zeros(1), None, g1, np.zeros(1), np.zeros(1), hp, 1,
                                        "fp32", v_dtype="fp16")
    assert v1[0] == 0.0
    p2, _, m2, v2 = O.adamw_step_stored(p1, None, np.zeros(1), m1, v1, hp, 2, "fp32",
                                        v_dtype="fp16")
    m_hat = 0.9 * m1[0] / (1 - 0.9 ** 2)
    assert p2[0] - p1[0] == pytest.approx(-1e-3 * m_hat / 1e-8, rel=1e-6)
    # with fp32 v the same step is of order lr
    q1, _, n1, w1 = O.adamw_step_stored(np.zeros(1), None, g1, np.zeros(1), np.zeros(1), hp, 1,
                                        "fp32")
    q2, _, _, _ = O.adamw_step_stored(q1, None, np.zeros(1), n1, w1, hp, 2, "fp32")
    assert abs(q2[0] - q1[0]) < 2e-3


def test_state_bytes():
    assert O.adamw_state_bytes_per_param() == 8
    assert O.adamw_state_bytes_per_param("bf16", "fp16") == 4
    assert O.adamw_state_bytes_per_param("fp32", "bf16") == 6
