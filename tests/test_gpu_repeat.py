"""Run-to-run determinism of the float outputs: every kernel of the library sums in a
fixed order (no atomics), so the same call on the same inputs gives the same bits.
Each entry point is called twice (decode calls on fresh copies of the caches, which
they write) and the two outputs must be equal bit for bit."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from synth import bf16_round
from synth.workloads import attn_case, ffn_case, layer_case
from tests._gpu import bf16, dev, log, nan_bf16, needs_gpu, u8
from tests.test_gpu_layer import gpu_weights


def _same(a: torch.Tensor, b: torch.Tensor):
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "two runs differ"


@needs_gpu
@pytest.mark.parametrize("mode,T", [("prefill", 700), ("decode", 24), ("decode", 64)])
def test_ffn_repeats_bitwise(mode, T):
    dev()
    log(f"repeat ffn {mode} T={T}")
    c = ffn_case(f"rep_ffn_{mode}_{T}", T, 512, 2048, 16, 0.5, "bernoulli")
    args = (bf16(c["X"]), u8(c["mask"]), bf16(c["W_gate"]), bf16(c["W_up"]),
            wide.pack_kmajor(bf16(c["W_down"]), 16))
    ys = [wide.ffn_masked(*args, mode=mode, out=nan_bf16((T, 512))) for _ in range(2)]
    _same(*ys)


@needs_gpu
def test_attention_prefill_repeats_bitwise():
    dev()
    log("repeat attention prefill")
    c = attn_case("rep_attn", 600, 512, 16, 4, 128, 0.5, "bernoulli")
    args = (bf16(c["X"]), u8(c["mask"]), bf16(c["Wq"]), bf16(c["Wk"]), bf16(c["Wv"]),
            wide.pack_kmajor(bf16(c["Wo"]), 4))
    ys = [wide.attn_proj_masked(*args, n_q=16, n_kv=4, rope_theta=500000.0,
                                out=nan_bf16((600, 512))) for _ in range(2)]
    _same(*ys)


@needs_gpu
def test_attention_decode_repeats_bitwise():
    dev()
    log("repeat attention decode")
    B, L = 12, 700
    c = attn_case("rep_attn_dec", B, 512, 16, 4, 128, 0.5, "topk", decode=True, kv_len=L,
                  kv_cap=L + 1)
    args = (bf16(c["X"]), u8(c["mask"]), bf16(c["Wq"]), bf16(c["Wk"]), bf16(c["Wv"]),
            wide.pack_kmajor(bf16(c["Wo"]), 4))
    outs = []
    for _ in range(2):
        Kc, Vc = bf16(c["K_cache"]), bf16(c["V_cache"])
        outs.append((wide.attn_proj_masked(*args, n_q=16, n_kv=4, rope_theta=500000.0,
                                           mode="decode", K_cache=Kc, V_cache=Vc, kv_len=L,
                                           out=nan_bf16((B, 512))), Kc, Vc))
    for a, b in zip(*outs):
        _same(a, b)


@needs_gpu
@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_layer_repeats_bitwise(mode):
    dev()
    log(f"repeat layer {mode}")
    dec = mode == "decode"
    T, L = (20, 300) if dec else (520, 0)
    c = layer_case(f"rep_layer_{mode}", T, 512, 2048, 16, 16, 4, 128, 0.5, "router", decode=dec,
                   kv_len=L, kv_cap=L + 1 if dec else 0)
    W = gpu_weights(c)
    outs = []
    for _ in range(2):
        kw = {}
        if dec:
            kw = dict(mode="decode", K_cache=bf16(c["K_cache"]), V_cache=bf16(c["V_cache"]),
                      kv_len=L)
        outs.append(wide.layer_masked(bf16(c["X"]), u8(c["attn_mask"]), u8(c["ffn_mask"]), W,
                                      n_q=16, n_kv=4, rope_theta=500000.0, eps=1e-5,
                                      out=nan_bf16((T, 512)), **kw))
    _same(*outs)


@needs_gpu
def test_router_repeats_bitwise():
    dev()
    log("repeat router")
    T, d, n = 1000, 512, 112
    X = bf16(bf16_round(np.random.default_rng(1).standard_normal((T, d))))
    R = wide.pack_router(bf16(bf16_round(np.random.default_rng(2).standard_normal((n, d)))))
    a = wide.router_topk(X, R, 56, n, return_logits=True)
    b = wide.router_topk(X, R, 56, n, return_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(a["logits"], b["logits"]) and torch.equal(a["mask"], b["mask"])
