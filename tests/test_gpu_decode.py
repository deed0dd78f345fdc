"""GPU parity of the decode paths (a batch of single tokens against K/V caches):
wide_ffn_masked(mode=decode), wide_attn_proj_masked(mode=decode) including the
cache writes, and wide_layer_masked(mode=decode)."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import attn_masked, ffn_masked, layer_masked
from synth import bf16_round
from synth.workloads import attn_case, attn_decode_8b, ffn_case, ffn_decode_8b, layer_8b, layer_case
from tests._gpu import TOL, bf16, dev, host, log, nan_bf16, needs_gpu, rel_err, u8
from tests.test_gpu_layer import gpu_weights


def _gpu_ffn(c, mode):
    n = c["mask"].shape[1]
    T, d = c["X"].shape
    Y = nan_bf16((T, d))
    wide.ffn_masked(bf16(c["X"]), u8(c["mask"]), bf16(c["W_gate"]), bf16(c["W_up"]),
                    wide.pack_kmajor(bf16(c["W_down"]), n), mode=mode, out=Y)
    torch.cuda.synchronize()
    return host(Y)


@needs_gpu
@pytest.mark.parametrize("B,d,F,n,kind", [(1, 512, 2048, 16, "topk"), (5, 256, 1024, 8, "bernoulli"),
                                          (17, 384, 1536, 12, "topk"), (64, 256, 2048, 32, "clustered"),
                                          (33, 256, 1024, 8, "ones"), (9, 256, 1024, 8, "zeros"),
                                          (100, 256, 1024, 8, "topk"), (24, 128, 512, 8, "topk"),
                                          (48, 448, 1024, 16, "bernoulli"),
                                          (8, 256, 512, 16, "topk"), (40, 384, 1024, 32, "bernoulli"),
                                          (2, 256, 1024, 16, "topk"), (4, 256, 1024, 8, "zeros"),
                                          (3, 384, 1536, 24, "clustered")])
def test_ffn_decode_shapes(B, d, F, n, kind):
    dev()
    log(f"ffn decode B={B} d={d} F={F} n={n} {kind}")
    c = ffn_case(f"ffn_dec_{B}_{d}_{kind}", B, d, F, n, 0.5, kind)
    got = _gpu_ffn(c, "decode")
    ref = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"])
    assert rel_err(got, ref) <= TOL


@needs_gpu
@pytest.mark.parametrize("B", [1, 8, 32, 64])
def test_ffn_decode_llama31_8b(B):
    """Llama-3.1-8B FFN decode: d=4096, d_ff=14336 in 112 groups, keep 56."""
    dev()
    log(f"ffn decode 8B B={B}")
    c = ffn_decode_8b(B)
    got = _gpu_ffn(c, "decode")
    ref = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"])
    assert rel_err(got, ref) <= TOL


def _gpu_attn_decode(c, theta):
    m = c["meta"]
    B, d = c["X"].shape
    Kc, Vc = bf16(c["K_cache"]), bf16(c["V_cache"])
    Y = nan_bf16((B, d))
    wide.attn_proj_masked(bf16(c["X"]), u8(c["mask"]), bf16(c["Wq"]), bf16(c["Wk"]), bf16(c["Wv"]),
                          wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]), n_q=m["n_q"], n_kv=m["n_kv"],
                          rope_theta=theta, mode="decode", K_cache=Kc, V_cache=Vc,
                          kv_len=m["kv_len"], out=Y)
    torch.cuda.synchronize()
    return host(Y), host(Kc), host(Vc)


def _check_attn_decode(c, theta):
    m = c["meta"]
    L = m["kv_len"]
    Y, Kg, Vg = _gpu_attn_decode(c, theta)
    Yr, Kn, Vn = attn_masked(c["X"], c["mask"], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                             n_kv=m["n_kv"], head_dim=128, rope_theta=theta, decode=True,
                             K_cache=c["K_cache"], V_cache=c["V_cache"], kv_len=L)
    assert rel_err(Y, Yr) <= TOL
    keep = c["mask"] != 0
    # the new token's k/v land in slot kv_len of the kept (token, group) pairs only
    assert rel_err(Kg[:, :, L][keep], Kn[keep]) <= TOL
    assert rel_err(Vg[:, :, L][keep], Vn[keep]) <= TOL
    K0, V0 = c["K_cache"].copy(), c["V_cache"].copy()
    K0[:, :, L][keep] = Kg[:, :, L][keep]
    V0[:, :, L][keep] = Vg[:, :, L][keep]
    assert np.array_equal(Kg, K0) and np.array_equal(Vg, V0), "cache written outside kept slots"


ATT = [
    # B, d, n_q, n_kv, kv_len, kv_cap, keep, kind, theta
    (1, 256, 8, 2, 0, 1, 0.5, "ones", 0.0),
    (3, 256, 8, 2, 1, 5, 0.5, "bernoulli", 500000.0),
    (5, 256, 16, 4, 255, 300, 0.5, "topk", 500000.0),
    (4, 256, 8, 2, 256, 257, 0.5, "bernoulli", 0.0),
    (7, 384, 12, 4, 700, 1024, 0.5, "topk", 10000.0),     # r = 3
    (2, 256, 16, 2, 300, 301, 0.75, "bernoulli", 0.0),    # r = 8
    (16, 256, 8, 8, 1000, 1001, 0.5, "clustered", 500000.0),
    (6, 256, 8, 2, 99, 100, 0.0, "zeros", 500000.0),
    (40, 320, 8, 2, 130, 131, 0.5, "topk", 500000.0),     # batch over 16: LDS-shared rows
    (20, 128, 8, 4, 10, 12, 0.5, "bernoulli", 0.0),       # d below one 256-wide K batch
    (64, 512, 16, 4, 33, 40, 0.75, "clustered", 10000.0),
    (48, 256, 16, 16, 140, 141, 0.5, "topk", 500000.0),   # r = 1, 16 groups
    (2, 256, 8, 2, 16500, 16501, 0.5, "topk", 500000.0),  # over 128 key chunks
]


@needs_gpu
@pytest.mark.parametrize("B,d,n_q,n_kv,L,cap,keep,kind,theta", ATT)
def test_attn_decode_shapes(B, d, n_q, n_kv, L, cap, keep, kind, theta):
    dev()
    log(f"attn decode B={B} d={d} n_q={n_q} n_kv={n_kv} L={L} cap={cap} {kind} theta={theta}")
    c = attn_case(f"attn_dec_{B}_{L}_{kind}", B, d, n_q, n_kv, 128, keep, kind, decode=True,
                  kv_len=L, kv_cap=cap)
    _check_attn_decode(c, theta)


@needs_gpu
def test_attn_decode_llama31_8b_full():
    """Llama-3.1-8B attention decode: batch 16 over a 4096-entry cache, keep 4 of 8."""
    dev()
    log("attn decode 8B B=16 L=4096")
    _check_attn_decode(attn_decode_8b(), 0.0)


@needs_gpu
def test_attn_decode_matches_prefill_row():
    """All-ones masks: decoding token L against the oracle's (bf16) K/V of tokens
    0..L-1 reproduces row L of the oracle prefill over L+1 tokens."""
    dev()
    L, d, n_q, n_kv, theta = 300, 256, 8, 2, 500000.0
    c = attn_case("attn_dec_chain", L + 1, d, n_q, n_kv, 128, 1.0, "ones")
    Yp = attn_masked(c["X"], c["mask"], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=n_q, n_kv=n_kv,
                     head_dim=128, rope_theta=theta)
    from oracle import rope
    X = c["X"]
    k = rope((X @ c["Wk"].T).reshape(L + 1, n_kv, 128), np.arange(L + 1), theta)
    v = (X @ c["Wv"].T).reshape(L + 1, n_kv, 128)
    Kc = np.zeros((1, n_kv, L + 1, 128), np.float32)
    Vc = np.zeros((1, n_kv, L + 1, 128), np.float32)
    Kc[0, :, :L] = bf16_round(k[:L].transpose(1, 0, 2).astype(np.float32))
    Vc[0, :, :L] = bf16_round(v[:L].transpose(1, 0, 2).astype(np.float32))
    dc = dict(c, X=X[L:], mask=c["mask"][L:], K_cache=Kc, V_cache=Vc,
              meta=dict(c["meta"], kv_len=L, kv_cap=L + 1))
    Y, _, _ = _gpu_attn_decode(dc, theta)
    assert rel_err(Y[0], Yp[L]) <= TOL


def _gpu_layer_decode(c):
    m = c["meta"]
    B, d = c["X"].shape
    Kc, Vc = bf16(c["K_cache"]), bf16(c["V_cache"])
    Y = nan_bf16((B, d))
    wide.layer_masked(bf16(c["X"]), u8(c["attn_mask"]), u8(c["ffn_mask"]), gpu_weights(c),
                      n_q=m["n_q"], n_kv=m["n_kv"], rope_theta=m["rope_theta"], eps=m["eps"],
                      mode="decode", K_cache=Kc, V_cache=Vc, kv_len=m["kv_len"], out=Y)
    torch.cuda.synchronize()
    return host(Y), host(Kc), host(Vc)


def _oracle_layer_decode(c):
    m = c["meta"]
    return layer_masked(c["X"], c["attn_mask"], c["ffn_mask"], c, n_q=m["n_q"], n_kv=m["n_kv"],
                        head_dim=128, n_ffn=m["n_ffn"], rope_theta=m["rope_theta"], eps=m["eps"],
                        decode=True, K_cache=c["K_cache"], V_cache=c["V_cache"], kv_len=m["kv_len"],
                        return_parts=True)


def _check_layer_decode(c):
    """y against the oracle, and what y hides behind the residual x: the layer's
    own cache writes (slot kv_len of the kept pairs only), its update y - x against
    the oracle's attention-plus-FFN term (bound: the tolerance on that term plus the
    bf16 roundings of h and y), and each sublayer alone on the oracle's bf16-rounded
    intermediate input (u for attention, w for the FFN)."""
    m = c["meta"]
    L = m["kv_len"]
    y, Kg, Vg = _gpu_layer_decode(c)
    ref, parts = _oracle_layer_decode(c)
    assert rel_err(y, ref) <= TOL
    keep = c["attn_mask"] != 0
    assert rel_err(Kg[:, :, L][keep], parts["K_new"][keep]) <= TOL
    assert rel_err(Vg[:, :, L][keep], parts["V_new"][keep]) <= TOL
    K0, V0 = c["K_cache"].copy(), c["V_cache"].copy()
    K0[:, :, L][keep] = Kg[:, :, L][keep]
    V0[:, :, L][keep] = Vg[:, :, L][keep]
    assert np.array_equal(Kg, K0) and np.array_equal(Vg, V0), "cache written outside kept slots"
    # the layer rounds h = x + a and y to bf16 (half an ulp each, 2^-9 relative)
    delta = parts["a"] + parts["f"]
    bound = TOL * np.abs(delta).max() + 2.0 ** -8 * (np.abs(parts["h"]).max() + np.abs(ref).max())
    assert np.abs((y - c["X"]) - delta).max() <= bound
    # attention sublayer alone on u (same caches, same slot), FFN sublayer alone on w
    u = bf16_round(parts["u"].astype(np.float32))
    ca = dict(c, X=u, mask=c["attn_mask"])
    _check_attn_decode(ca, m["rope_theta"])
    w = bf16_round(parts["w"].astype(np.float32))
    cf = dict(X=w, mask=c["ffn_mask"], W_gate=c["W_gate"], W_up=c["W_up"], W_down=c["W_down"])
    assert rel_err(_gpu_ffn(cf, "decode"),
                   ffn_masked(w, c["ffn_mask"], c["W_gate"], c["W_up"], c["W_down"])) <= TOL


@needs_gpu
@pytest.mark.parametrize("B,L,kind", [(4, 37, "router"), (32, 600, "bernoulli"), (9, 255, "clustered")])
def test_layer_decode_shapes(B, L, kind):
    dev()
    log(f"layer decode B={B} L={L} {kind}")
    c = layer_case(f"layer_dec_{B}_{L}_{kind}", B, 256, 1024, 8, 8, 2, 128, 0.5, kind,
                   decode=True, kv_len=L, kv_cap=L + 3)
    _check_layer_decode(c)


@needs_gpu
@pytest.mark.parametrize("kind,keep,attn_keep", [("router", 0.5, None), ("clustered", 0.5, None),
                                                 ("router", 0.72, 0.34)])
def test_layer_decode_llama31_8b_full(kind, keep, attn_keep):
    """Llama-3.1-8B layer decode at batch 32 over an 8192-entry cache: router top-k masks
    at 50 %, clustered masks, and the asymmetric keep (3 of 8 head groups, 81 of 112 FFN
    groups)."""
    dev()
    log(f"layer decode 8B B=32 L=8192 {kind} keep={keep} attn_keep={attn_keep}")
    c = layer_8b(32, decode=True, L=8192, kind=kind, keep=keep, attn_keep=attn_keep)
    _check_layer_decode(c)
