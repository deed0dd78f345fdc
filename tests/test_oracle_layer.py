"""Pins of the oracle's masked decoder layer (reading R6).

All-ones masks: the layer equals transformers' dense LlamaDecoderLayer in
float64 (RMSNorm, rotate-half RoPE with theta, GQA, SwiGLU).  All-zero masks:
y == x exactly, because both sublayers add an exact zero.  Mixed masks (one
sublayer all-ones, the other all-zero): y equals the library's other sublayer
with its residual alone.  RMSNorm against torch.nn.functional.rms_norm.
"""
import numpy as np
import pytest
import torch

from oracle import layer_masked, rmsnorm
from tests._libref import llama_layer, t64


def _weights(d, F, n_q, n_kv, hd, seed):
    r = np.random.default_rng(seed)
    s = 0.2
    return dict(Wq=r.standard_normal((n_q * hd, d)) * s, Wk=r.standard_normal((n_kv * hd, d)) * s,
                Wv=r.standard_normal((n_kv * hd, d)) * s, Wo=r.standard_normal((n_q * hd, d)) * s,
                W_gate=r.standard_normal((F, d)) * s, W_up=r.standard_normal((F, d)) * s,
                W_down=r.standard_normal((F, d)) * s, rms1=1 + 0.1 * r.standard_normal(d),
                rms2=1 + 0.1 * r.standard_normal(d))


def test_rmsnorm_matches_torch():
    x = np.random.default_rng(0).standard_normal((9, 40)) * 3
    gam = np.random.default_rng(1).standard_normal(40)
    ref = torch.nn.functional.rms_norm(t64(x), (40,), t64(gam), eps=1e-5).numpy()
    np.testing.assert_allclose(rmsnorm(x, gam, 1e-5), ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("n_q,n_kv", [(4, 2), (8, 8)])
def test_all_ones_is_llama_layer(n_q, n_kv):
    T, d, F, hd, n_ffn = 19, 32, 48, 8, 6
    W = _weights(d, F, n_q, n_kv, hd, 2)
    X = np.random.default_rng(3).standard_normal((T, d))
    y = layer_masked(X, np.ones((T, n_kv), np.uint8), np.ones((T, n_ffn), np.uint8), W,
                     n_q=n_q, n_kv=n_kv, head_dim=hd, n_ffn=n_ffn, rope_theta=500000.0, eps=1e-5)
    ref = llama_layer(X, W, n_q, n_kv, hd, 500000.0, 1e-5)
    # transformers' rotary tables are float32 (angle error ~ T * 2^-23)
    np.testing.assert_allclose(y, ref, rtol=0, atol=50.0 * T * 2.0 ** -23)


def test_all_zero_masks_return_input_exactly():
    T, d, F, n_q, n_kv, hd, n_ffn = 11, 32, 64, 4, 2, 8, 8
    W = _weights(d, F, n_q, n_kv, hd, 4)
    X = np.random.default_rng(5).standard_normal((T, d))
    y = layer_masked(X, np.zeros((T, n_kv), np.uint8), np.zeros((T, n_ffn), np.uint8), W,
                     n_q=n_q, n_kv=n_kv, head_dim=hd, n_ffn=n_ffn, rope_theta=500000.0, eps=1e-5)
    np.testing.assert_array_equal(y, X)


def test_rows_option_selects_rows():
    T, d, F, n_q, n_kv, hd, n_ffn = 23, 32, 64, 4, 2, 8, 8
    W = _weights(d, F, n_q, n_kv, hd, 6)
    rr = np.random.default_rng(7)
    X = rr.standard_normal((T, d))
    am = (rr.random((T, n_kv)) < 0.5).astype(np.uint8)
    fm = (rr.random((T, n_ffn)) < 0.5).astype(np.uint8)
    kw = dict(n_q=n_q, n_kv=n_kv, head_dim=hd, n_ffn=n_ffn, rope_theta=500000.0, eps=1e-5)
    rows = np.array([1, 5, 22])
    full = layer_masked(X, am, fm, W, **kw)
    part = layer_masked(X, am, fm, W, rows=rows, **kw)
    np.testing.assert_allclose(part, full[rows], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("which", ["attn", "mlp"])
def test_mixed_masks_leave_one_library_sublayer(which):
    """Attention all-ones with the FFN all-zero gives x + attention(RMSNorm(x)); the
    FFN all-ones with attention all-zero gives x + MLP(RMSNorm(x)) (transformers'
    LlamaDecoderLayer pieces, float64)."""
    T, d, F, n_q, n_kv, hd, n_ffn = 17, 32, 48, 4, 2, 8, 6
    W = _weights(d, F, n_q, n_kv, hd, 8)
    X = np.random.default_rng(9).standard_normal((T, d))
    ones_a = which == "attn"
    am = np.full((T, n_kv), 1 if ones_a else 0, np.uint8)
    fm = np.full((T, n_ffn), 0 if ones_a else 1, np.uint8)
    y = layer_masked(X, am, fm, W, n_q=n_q, n_kv=n_kv, head_dim=hd, n_ffn=n_ffn,
                     rope_theta=500000.0, eps=1e-5)
    ref = llama_layer(X, W, n_q, n_kv, hd, 500000.0, 1e-5, part=which)
    np.testing.assert_allclose(y, ref, rtol=0, atol=50.0 * T * 2.0 ** -23)
