"""Pins of oracle/clip_oracle.py (MuonClip: Frobenius-norm clip of weight
blocks and the max-logit rescale of W_q / W_k) against closed forms, the
spectral-norm bound through an SVD, and the max logit of a small attention
head recomputed after the clip."""

import math

import numpy as np
import pytest

from oracle import clip_oracle as C
from oracle import muon_oracle as O


def test_frobenius_clip_diag_three_four():
    w = np.zeros(12)
    w[0], w[5] = 3.0, 4.0                      # 3 x 4 block, diag(3, 4): ||W||_F = 5
    out, norms, gammas = C.muon_clip_flat(w, [(0, 3, 4, 4, 0)], C.MODE_FROBENIUS, 1.0, None,
                                          "fp64")
    assert norms == [5.0] and gammas == [0.2]
    assert out[0] == pytest.approx(0.6, rel=1e-15) and out[5] == pytest.approx(0.8, rel=1e-15)
    assert np.linalg.norm(out) == pytest.approx(1.0, rel=1e-15)
    # the spectral norm, 4 before, is 0.8 after: <= tau
    assert np.linalg.svd(out.reshape(3, 4), compute_uv=False)[0] == pytest.approx(0.8, rel=1e-14)


def test_frobenius_clip_below_threshold_is_identity():
    rng = np.random.default_rng(0)
    w = rng.standard_normal(64)
    out, norms, gammas = C.muon_clip_flat(w, [(0, 8, 8, 8, 0)], C.MODE_FROBENIUS,
                                          float(np.linalg.norm(w)) * 1.0001, None, "fp64")
    assert gammas == [1.0] and np.array_equal(out, w)


def test_rank_one_block_spectral_equals_tau():
    # W = u v^T: spectral = Frobenius = |u||v|, so the clip lands exactly on tau
    u, v = np.array([1.0, -2.0, 2.0]), np.array([0.5, 0.5, 0.5, 0.5])
    w = np.outer(u, v).reshape(-1)
    out, norms, _ = C.muon_clip_flat(w, [(0, 3, 4, 4, 0)], C.MODE_FROBENIUS, 0.75, None, "fp64")
    assert norms[0] == pytest.approx(3.0, rel=1e-15)
    s = np.linalg.svd(out.reshape(3, 4), compute_uv=False)
    assert s[0] == pytest.approx(0.75, rel=1e-14) and s[1] < 1e-15


def test_spectral_bound_controls_xw():
    rng = np.random.default_rng(1)
    w = rng.standard_normal(40 * 24) * 3.0
    tau = 2.5
    out, norms, gammas = C.muon_clip_flat(w, [(0, 40, 24, 24, 0)], C.MODE_FROBENIUS, tau, None,
                                          "fp64")
    W = out.reshape(40, 24)
    assert gammas[0] < 1.0
    assert np.linalg.norm(W) == pytest.approx(tau, rel=1e-14)
    assert np.linalg.svd(W, compute_uv=False)[0] <= tau * (1 + 1e-14)
    x = rng.standard_normal((100, 24))
    # ||x W^T||_2 <= tau ||x||_2 row by row
    assert np.all(np.linalg.norm(x @ W.T, axis=1) <= tau * np.linalg.norm(x, axis=1) * (1 + 1e-13))


def test_strided_blocks_touch_only_their_elements():
    # two heads of 2 rows in a 6 x 5 matrix with ld 7 (a column pad of 2)
    rng = np.random.default_rng(2)
    flat = rng.standard_normal(3 + 6 * 7) * 5.0
    t0 = (3, 2, 5, 7, 0)              # rows 0-1
    t1 = (3 + 4 * 7, 2, 5, 7, 1)      # rows 4-5
    out, norms, gammas = C.muon_clip_flat(flat, [t0, t1], C.MODE_FROBENIUS, 1.0, None, "fp64")
    touched = np.zeros(flat.size, bool)
    for t in (t0, t1):
        idx, w = C.block_view(flat, t)
        touched[idx] = True
        assert np.linalg.norm(out[idx]) == pytest.approx(1.0, rel=1e-14)
    assert np.array_equal(out[~touched], flat[~touched])
    # the blocks' flat indices, written out by hand: rows 0-1 and 4-5 of a
    # matrix starting at 3 with 7 elements per row, first 5 columns
    want = [3, 4, 5, 6, 7, 10, 11, 12, 13, 14, 31, 32, 33, 34, 35, 38, 39, 40, 41, 42]
    assert np.flatnonzero(touched).tolist() == want


def test_attention_max_logit_by_hand():
    # x = I2, W_q = [1, 2], W_k = [3, -1]: q = (1, 2), k = (3, -1), logits
    # q_i k_j = [[3, -1], [6, -2]]: the largest is 6
    x = np.eye(2)
    assert C.attention_max_logit(x, np.array([[1.0, 2.0]]), np.array([[3.0, -1.0]])) == 6.0
    # W_q = I, W_k swaps the two features: q = x = [[1, 1], [2, -1]],
    # k = [[1, 1], [-1, 2]], logits [[2, 1], [1, -4]]: the largest is 2
    # (with k taken from W_q it would be 5)
    x = np.array([[1.0, 1.0], [2.0, -1.0]])
    assert C.attention_max_logit(x, np.eye(2), np.array([[0.0, 1.0], [1.0, 0.0]])) == 2.0


def _heads(rng, n_heads, d_head, d_model, scale):
    wq = rng.standard_normal((n_heads * d_head, d_model)) * scale
    wk = rng.standard_normal((n_heads * d_head, d_model)) * scale
    return wq, wk


def test_max_logit_mode_lands_on_tau():
    rng = np.random.default_rng(3)
    n_heads, d_head, d_model = 4, 8, 32
    wq, wk = _heads(rng, n_heads, d_head, d_model, 1.0)
    x = rng.standard_normal((16, d_model))
    S = [C.attention_max_logit(x, wq[h * d_head:(h + 1) * d_head], wk[h * d_head:(h + 1) * d_head])
         for h in range(n_heads)]
    tau = float(np.median(S))           # two heads over, two under
    flat = np.concatenate([wq.reshape(-1), wk.reshape(-1)])
    kofs = wq.size
    targets = []
    for h in range(n_heads):
        targets.append((h * d_head * d_model, d_head, d_model, d_model, h))
        targets.append((kofs + h * d_head * d_model, d_head, d_model, d_model, h))
    out, _, gammas = C.muon_clip_flat(flat, targets, C.MODE_MAX_LOGIT, tau, S, "fp64")
    wq2, wk2 = out[:kofs].reshape(wq.shape), out[kofs:].reshape(wk.shape)
    for h in range(n_heads):
        sl = slice(h * d_head, (h + 1) * d_head)
        s2 = C.attention_max_logit(x, wq2[sl], wk2[sl])
        if S[h] > tau:
            assert s2 == pytest.approx(tau, rel=1e-12)
            assert gammas[2 * h] == gammas[2 * h + 1] == pytest.approx(math.sqrt(tau / S[h]))
        else:
            assert s2 == S[h]
            assert np.array_equal(wq2[sl], wq[sl]) and np.array_equal(wk2[sl], wk[sl])


def test_logit_factor_cases():
    assert C.logit_clip_factor(400.0, 100.0) == 0.5
    assert C.logit_clip_factor(100.0, 100.0) == 1.0
    assert C.logit_clip_factor(-5.0, 100.0) == 1.0
    assert C.logit_clip_factor(math.nan, 100.0) == 1.0
    assert C.logit_clip_factor(math.inf, 100.0) == 1.0


def test_non_finite_and_zero_blocks_are_left_alone():
    w = np.array([np.nan, 1.0, 2.0, 3.0])
    _, norms, gammas = C.muon_clip_flat(w, [(0, 2, 2, 2, 0)], C.MODE_FROBENIUS, 1.0, None, "fp64")
    assert math.isnan(norms[0]) and gammas == [1.0]
    z = np.zeros(9)
    out, norms, gammas = C.muon_clip_flat(z, [(0, 3, 3, 3, 0)], C.MODE_FROBENIUS, 1.0, None, "fp64")
    assert norms == [0.0] and gammas == [1.0] and np.array_equal(out, z)
    with pytest.raises(ValueError):
        C.muon_clip_flat(z, [(0, 3, 3, 3, 0)], C.MODE_FROBENIUS, 0.0, None, "fp64")


def test_storage_rounding_matches_library_casts():
    # the rounded result is the library's RNE cast of gamma * w (fp64 -> fp32
    # is exact-then-round in both; bf16 through torch's own cast)
    import torch
    rng = np.random.default_rng(4)
    w = O.bf16_round(rng.standard_normal(300) * 4.0)
    for dt, tdt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
        out, _, gammas = C.muon_clip_flat(w, [(0, 10, 30, 30, 0)], C.MODE_FROBENIUS, 2.0, None, dt)
        want = torch.tensor(gammas[0] * w, dtype=torch.float64).to(torch.float32).to(tdt)
        assert np.array_equal(out, want.double().numpy())
