"""Pins of the oracle's masked SwiGLU FFN (gist.science §2.A; reading R2).

Checked against torch's own silu/matmul (an independent library formulation),
the exact zero of an all-zero mask, the per-token channel-subset form, group
additivity, a hand-worked fixture and brute force over all masks of a tiny case.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import ffn_masked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(T, d, F, n, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((T, d)), r.standard_normal((F, d)) * 0.3,
            r.standard_normal((F, d)) * 0.3, r.standard_normal((F, d)) * 0.3)


def _torch_dense(X, Wg, Wu, Wd):
    X, Wg, Wu, Wd = (torch.tensor(a, dtype=torch.float64) for a in (X, Wg, Wu, Wd))
    return (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T) @ Wd).numpy()


def test_golden_hand_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "ffn_2x2.json")))
    Y = ffn_masked(np.array(fx["X"]), np.array(fx["mask"]), np.array(fx["W_gate"]),
                   np.array(fx["W_up"]), np.array(fx["W_down"]))
    np.testing.assert_allclose(Y, np.array(fx["Y"]), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("T,d,F,n", [(7, 16, 32, 4), (33, 24, 48, 6), (64, 64, 256, 16)])
def test_all_ones_is_dense_swiglu(T, d, F, n):
    X, Wg, Wu, Wd = _case(T, d, F, n, 1)
    Y = ffn_masked(X, np.ones((T, n), np.uint8), Wg, Wu, Wd)
    np.testing.assert_allclose(Y, _torch_dense(X, Wg, Wu, Wd), rtol=1e-12, atol=1e-12)


def test_all_zero_is_exact_zero():
    X, Wg, Wu, Wd = _case(9, 16, 32, 4, 2)
    Y = ffn_masked(X, np.zeros((9, 4), np.uint8), Wg, Wu, Wd)
    assert np.all(Y == 0.0)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_per_token_channel_subset(seed):
    """Y[t] equals the dense FFN restricted to the channels of the groups t keeps
    (dropping a group = removing its channels; group g = channels gG..gG+G-1)."""
    T, d, F, n = 11, 20, 40, 5
    G = F // n
    X, Wg, Wu, Wd = _case(T, d, F, n, seed)
    m = (np.random.default_rng(seed).random((T, n)) < 0.5).astype(np.uint8)
    Y = ffn_masked(X, m, Wg, Wu, Wd)
    for t in range(T):
        ch = [c for c in range(F) if m[t, c // G]]
        ref = _torch_dense(X[t:t + 1], Wg[ch], Wu[ch], Wd[ch]) if ch else np.zeros((1, d))
        np.testing.assert_allclose(Y[t], ref[0], rtol=1e-12, atol=1e-12)


def test_disjoint_additivity():
    T, d, F, n = 17, 16, 48, 6
    X, Wg, Wu, Wd = _case(T, d, F, n, 6)
    r = np.random.default_rng(7)
    m = (r.random((T, n)) < 0.6).astype(np.uint8)
    split = (r.random((T, n)) < 0.5).astype(np.uint8)
    m1, m2 = m & split, m & (1 - split)
    y, y1, y2 = (ffn_masked(X, a, Wg, Wu, Wd) for a in (m, m1, m2))
    assert np.max(np.abs(y1 + y2 - y)) <= 1e-12 * np.max(np.abs(y))


def test_brute_force_all_masks():
    """d=8, d_ff=16, 4 groups, T=3: all 2^12 masks against the sum over kept
    (token, group) pairs of the one-group FFN computed by torch on weight slices."""
    T, d, F, n = 3, 8, 16, 4
    G = F // n
    X, Wg, Wu, Wd = _case(T, d, F, n, 8)
    f = np.zeros((T, n, d))
    for t in range(T):
        for g in range(n):
            s = slice(g * G, (g + 1) * G)
            f[t, g] = _torch_dense(X[t:t + 1], Wg[s], Wu[s], Wd[s])[0]
    for bits in itertools.product((0, 1), repeat=T * n):
        m = np.array(bits, np.uint8).reshape(T, n)
        Y = ffn_masked(X, m, Wg, Wu, Wd)
        ref = np.einsum("tg,tgd->td", m.astype(np.float64), f)
        assert np.max(np.abs(Y - ref)) <= 1e-12
