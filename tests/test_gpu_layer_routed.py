"""GPU parity of the router-fed path: wide_mask_reorder_packed (the reorder started from
the router's packed words) and wide_layer_masked_routed (two linear routers on the layer
input choose the masks, whose packed words go straight to the reorders).

The selection is an integer decision taken on floating point: the routed layer's masks
must equal, bit for bit, those of wide_router_topk on the same input (the same kernel),
whose selection the oracle checks on the logits the GPU returned (reading R9).  The layer
output is then checked against the oracle layer with those masks."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import layer_masked, mask_reorder, router_topk
from synth import normal
from synth.workloads import layer_8b, layer_case
from tests._gpu import TOL, bf16, dev, host, log, nan_bf16, needs_gpu, rel_err, u8
from tests.test_gpu_layer import gpu_weights


@needs_gpu
@pytest.mark.parametrize("T,n,tile_m", [(1000, 8, 256), (8192, 112, 256), (777, 200, 64)])
def test_reorder_from_packed_words(T, n, tile_m):
    """The reorder from the router's packed words equals the oracle's reorder of the
    router's mask bytes."""
    dev()
    log(f"reorder from packed words T={T} n={n}")
    d = 256
    X = normal(f"rpk_{T}_{n}", "X", (T, d))
    R = normal(f"rpk_{T}_{n}", "R", (n, d), 1.0 / 64)
    out = wide.router_topk(bf16(X), wide.pack_router(bf16(R)), n // 2, n)
    ro = wide.mask_reorder_packed(out["packed"], n, tile_m)
    torch.cuda.synchronize()
    ref = mask_reorder(host(out["mask"]), tile_m)
    for k in ("group_count", "group_perm", "group_rank", "tile_count", "tile_groups"):
        assert np.array_equal(host(ro[k]), ref[k]), k


def _routers(c, tag, n_kv, n_ffn, d):
    R_attn = normal(tag, "R_attn", (n_kv, d), 1.0 / 64)
    R_ffn = normal(tag, "R_ffn", (n_ffn, d), 1.0 / 64)
    return R_attn, R_ffn


def _check_masks(X, R, k, got_mask):
    """got_mask == the standalone router's mask (bit for bit), whose selection equals
    the oracle's on the GPU's logits."""
    out = wide.router_topk(bf16(X), wide.pack_router(bf16(R)), k, R.shape[0], return_logits=True)
    torch.cuda.synchronize()
    ref = host(out["mask"])
    assert np.array_equal(host(got_mask), ref)
    sel = np.unique(np.linspace(0, X.shape[0] - 1, 48).astype(int))
    on_gpu_logits = router_topk(None, None, k, logits=host(out["logits"])[sel])
    assert np.array_equal(ref[sel], on_gpu_logits["mask"])
    return ref


def _routed(c, R_attn, R_ffn, k_attn, k_ffn, **kw):
    m = c["meta"]
    T, d = c["X"].shape
    Y = nan_bf16((T, d))
    Y, am, fm = wide.layer_masked_routed(
        bf16(c["X"]), wide.pack_router(bf16(R_attn)), k_attn, wide.pack_router(bf16(R_ffn)),
        k_ffn, gpu_weights(c), n_q=m["n_q"], n_kv=m["n_kv"], n_ffn=m["n_ffn"],
        rope_theta=m["rope_theta"], eps=m["eps"], out=Y, **kw)
    torch.cuda.synchronize()
    return Y, am, fm


@needs_gpu
@pytest.mark.parametrize("T,d,F,n_ffn,n_q,n_kv,k_attn,k_ffn", [
    (300, 256, 1024, 8, 8, 2, 1, 4),
    (513, 512, 2048, 16, 16, 4, 2, 8),
    (200, 256, 2048, 64, 8, 8, 3, 45),
])
def test_routed_layer_prefill(T, d, F, n_ffn, n_q, n_kv, k_attn, k_ffn):
    dev()
    log(f"routed layer prefill T={T} d={d} n_ffn={n_ffn} n_kv={n_kv}")
    tag = f"routed_{T}_{d}_{n_ffn}"
    c = layer_case(tag, T, d, F, n_ffn, n_q, n_kv, 128, 0.5, "router")
    R_attn, R_ffn = _routers(c, tag, n_kv, n_ffn, d)
    Y, am, fm = _routed(c, R_attn, R_ffn, k_attn, k_ffn)
    attn_mask = _check_masks(c["X"], R_attn, k_attn, am)
    ffn_mask = _check_masks(c["X"], R_ffn, k_ffn, fm)
    assert (attn_mask.sum(1) == k_attn).all() and (ffn_mask.sum(1) == k_ffn).all()
    m = c["meta"]
    ref = layer_masked(c["X"], attn_mask, ffn_mask, c, n_q=n_q, n_kv=n_kv, head_dim=128,
                       n_ffn=n_ffn, rope_theta=m["rope_theta"], eps=m["eps"])
    assert rel_err(host(Y), ref) <= TOL
    # the same masks through wide_layer_masked: the same kernels, the same output
    Y2 = nan_bf16((T, d))
    wide.layer_masked(bf16(c["X"]), u8(attn_mask), u8(ffn_mask), gpu_weights(c), n_q=n_q,
                      n_kv=n_kv, rope_theta=m["rope_theta"], eps=m["eps"], out=Y2)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))


@needs_gpu
def test_routed_layer_prefill_ffn_token_sort_bit_identical():
    """The router-fed layer with the FFN token sort (WIDE_FLAG_FFN_TOKEN_SORT; the
    sort keys come from the router's packed words): the same masks and the same
    output bit for bit as without it."""
    dev()
    T, d, F, n_ffn, n_q, n_kv = 700, 256, 2048, 16, 8, 2
    log(f"routed layer prefill T={T} n_ffn={n_ffn} with the FFN token sort")
    tag = "routed_sort"
    c = layer_case(tag, T, d, F, n_ffn, n_q, n_kv, 128, 0.5, "router")
    R_attn, R_ffn = _routers(c, tag, n_kv, n_ffn, d)
    Y0, am0, fm0 = _routed(c, R_attn, R_ffn, 1, 8)
    Y1, am1, fm1 = _routed(c, R_attn, R_ffn, 1, 8, sort_ffn_tokens=True)
    assert torch.equal(am0, am1) and torch.equal(fm0, fm1)
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))


@needs_gpu
def test_routed_layer_prefill_llama31_8b_sampled():
    """Llama-3.1-8B layer at T = 8192 with the routers on the GPU (keep 4 of 8 head
    groups and 56 of 112 FFN groups): masks bit-exact against the standalone router,
    24 sampled rows against the oracle."""
    dev()
    log("routed layer prefill 8B T=8192 (sampled)")
    c = layer_8b(8192)
    m = c["meta"]
    R_attn, R_ffn = _routers(c, "routed_8b", 8, 112, 4096)
    Y, am, fm = _routed(c, R_attn, R_ffn, 4, 56)
    attn_mask = _check_masks(c["X"], R_attn, 4, am)
    ffn_mask = _check_masks(c["X"], R_ffn, 56, fm)
    rows = np.sort(np.random.default_rng(4).choice(8192, 24, replace=False))
    rows[0], rows[-1] = 0, 8191
    ref = layer_masked(c["X"], attn_mask, ffn_mask, c, n_q=32, n_kv=8, head_dim=128, n_ffn=112,
                       rope_theta=m["rope_theta"], eps=m["eps"], rows=rows)
    got = host(Y)
    assert np.all(np.isfinite(got))
    assert rel_err(got[rows], ref) <= TOL


@needs_gpu
def test_routed_layer_decode():
    """Decode mode: the routers pick each new token's groups; the layer with those masks
    and the cache writes match the oracle."""
    dev()
    B, L, d, F, n_ffn, n_q, n_kv = 9, 130, 256, 1024, 8, 8, 2
    log(f"routed layer decode B={B} L={L}")
    tag = "routed_dec"
    c = layer_case(tag, B, d, F, n_ffn, n_q, n_kv, 128, 0.5, "router", decode=True, kv_len=L,
                   kv_cap=L + 2)
    m = c["meta"]
    R_attn, R_ffn = _routers(c, tag, n_kv, n_ffn, d)
    Kc, Vc = bf16(c["K_cache"]), bf16(c["V_cache"])
    Y, am, fm = _routed(c, R_attn, R_ffn, 1, 4, mode="decode", K_cache=Kc, V_cache=Vc, kv_len=L)
    attn_mask = _check_masks(c["X"], R_attn, 1, am)
    ffn_mask = _check_masks(c["X"], R_ffn, 4, fm)
    ref, parts = layer_masked(c["X"], attn_mask, ffn_mask, c, n_q=n_q, n_kv=n_kv, head_dim=128,
                              n_ffn=n_ffn, rope_theta=m["rope_theta"], eps=m["eps"], decode=True,
                              K_cache=c["K_cache"], V_cache=c["V_cache"], kv_len=L,
                              return_parts=True)
    assert rel_err(host(Y), ref) <= TOL
    keep = attn_mask != 0
    Kg = host(Kc)
    assert rel_err(Kg[:, :, L][keep], parts["K_new"][keep]) <= TOL
