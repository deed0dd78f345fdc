"""Calls recorded into a HIP graph (torch.cuda.graph) replay to the eager result bit
for bit: the layer (prefill and decode) and every decode entry point (FFN,
attention over a full, a masked and a paged cache, and the layer over a masked or
paged cache), which is how a serving loop launches a decode step.  Every call
launches its kernels on the caller's stream only, with no memset nodes; a decode
replay writes the new K/V into the same cache slots as the eager call.  Each
replay is preceded by eager work on the same buffers (a fill of the output, an
eager call into another output with the same workspace) and checked on its own."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from synth.workloads import attn_case, ffn_case, layer_case, paged_cache
from tests._gpu import bf16, dev, log, nan_bf16, needs_gpu, u8
from tests.test_gpu_layer import gpu_weights


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@needs_gpu
@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_layer_graph_replays_match_eager(mode):
    dev()
    log(f"graph capture layer {mode}")
    dec = mode == "decode"
    T, L = (24, 200) if dec else (300, 0)
    c = layer_case(f"graph_{mode}", T, 256, 1024, 8, 8, 2, 128, 0.5, "router", decode=dec,
                   kv_len=L, kv_cap=L + 1 if dec else 0)
    m = c["meta"]
    W = gpu_weights(c)
    X, am, fm = bf16(c["X"]), u8(c["attn_mask"]), u8(c["ffn_mask"])
    kw = dict(n_q=m["n_q"], n_kv=m["n_kv"], rope_theta=m["rope_theta"], eps=m["eps"], mode=mode)
    if dec:
        K, V = bf16(c["K_cache"]), bf16(c["V_cache"])
        kw.update(K_cache=K, V_cache=V, kv_len=L)
    ws = torch.empty(wide.layer_masked_workspace(T, 256, 1024, 8, m["n_q"], m["n_kv"], mode=mode,
                                                 kv_cap=L + 1 if dec else 0),
                     dtype=torch.uint8, device="cuda")
    ref = nan_bf16((T, 256))
    wide.layer_masked(X, am, fm, W, out=ref, workspace=ws, **kw)
    torch.cuda.synchronize()
    if dec:
        Kref, Vref = K.clone(), V.clone()

    Y = nan_bf16((T, 256))
    other = nan_bf16((T, 256))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # a call on the capture stream before capture
        wide.layer_masked(X, am, fm, W, out=Y, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wide.layer_masked(X, am, fm, W, out=Y, workspace=ws, **kw)
    torch.cuda.synchronize()
    for i in range(4):
        Y.fill_(float("nan"))
        wide.layer_masked(X, am, fm, W, out=other, workspace=ws, **kw)  # eager, same workspace
        g.replay()
        torch.cuda.synchronize()
        assert _same(Y, ref), f"replay {i} differs from the eager call"
        assert _same(other, ref)
        if dec:
            assert _same(K, Kref) and _same(V, Vref)


def _replays_match(shape, call, outs):
    """call(out) runs the entry point into `out` (of `shape`); outs: the buffers it
    also writes (caches), compared after every replay with their state after the
    eager call."""
    ref = nan_bf16(shape)
    call(ref)
    torch.cuda.synchronize()
    after = [o.clone() for o in outs]
    Y, other = nan_bf16(shape), nan_bf16(shape)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(Y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(Y)
    torch.cuda.synchronize()
    for i in range(4):
        Y.fill_(float("nan"))
        call(other)
        g.replay()
        torch.cuda.synchronize()
        assert _same(Y, ref), f"replay {i} differs from the eager call"
        assert _same(other, ref)
        for o, a in zip(outs, after):
            assert _same(o, a), f"replay {i} wrote the caches differently"


@needs_gpu
@pytest.mark.parametrize("entry", ["ffn", "attn", "attn_masked_cache", "attn_paged",
                                   "layer_masked_cache", "layer_paged"])
def test_decode_graph_replays_match_eager(entry):
    dev()
    log(f"graph capture decode {entry}")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev())
    if entry == "ffn":
        B, d = 20, 256
        c = ffn_case("graph_ffn_dec", B, d, 1024, 8, 0.5, "topk")
        X, mk = bf16(c["X"]), u8(c["mask"])
        Wg, Wu, Wd = bf16(c["W_gate"]), bf16(c["W_up"]), wide.pack_kmajor(bf16(c["W_down"]), 8)
        ws = torch.empty(wide.ffn_masked_workspace(B, d, 1024, 8, mode="decode"),
                         dtype=torch.uint8, device="cuda")
        _replays_match((B, d), lambda out: wide.ffn_masked(
            X, mk, Wg, Wu, Wd, mode="decode", out=out, workspace=ws), [])
        return
    B, d, nq, nkv, L = 12, 256, 8, 2, 300
    if entry.startswith("attn"):
        c = attn_case(f"graph_{entry}", B, d, nq, nkv, 128, 0.5, "topk", decode=True, kv_len=L,
                      kv_cap=L + 1)
        X, mk = bf16(c["X"]), u8(c["mask"])
        W = (bf16(c["Wq"]), bf16(c["Wk"]), bf16(c["Wv"]), wide.pack_kmajor(bf16(c["Wo"]), nkv))
        kw = dict(n_q=nq, n_kv=nkv, rope_theta=500000.0)
        ws = torch.empty(wide.attn_proj_masked_workspace(B, d, nq, nkv, mode="decode",
                                                         kv_cap=L + 1),
                         dtype=torch.uint8, device="cuda")
        lens = i32(np.random.default_rng(5).integers(0, L + 1, size=(B, nkv)))
        if entry == "attn":
            K, V = bf16(c["K_cache"]), bf16(c["V_cache"])
            fn = lambda out: wide.attn_proj_masked(X, mk, *W, mode="decode", K_cache=K, V_cache=V,
                                                   kv_len=L, out=out, workspace=ws, **kw)
            caches = [K, V]
        elif entry == "attn_masked_cache":
            K, V = bf16(c["K_cache"]), bf16(c["V_cache"])
            fn = lambda out: wide.attn_decode_masked_cache(X, mk, *W, K_cache=K, V_cache=V,
                                                           kv_len=lens, pos=L, out=out,
                                                           workspace=ws, **kw)
            caches = [K, V]
        else:
            p = paged_cache(f"graph_{entry}", B, nkv, 16, 20)
            Kp, Vp = bf16(p["K_pool"]), bf16(p["V_pool"])
            tab, pl = i32(p["page_table"]), i32(p["kv_len"])
            fn = lambda out: wide.attn_decode_masked_paged(X, mk, *W, K_pool=Kp, V_pool=Vp,
                                                           page_table=tab, kv_len=pl, pos=319,
                                                           out=out, **kw)
            caches = [Kp, Vp]
        _replays_match((B, d), fn, caches)
        return
    c = layer_case(f"graph_{entry}", B, d, 1024, 8, nq, nkv, 128, 0.5, "router", decode=True,
                   kv_len=L, kv_cap=L + 1)
    m = c["meta"]
    Wl = gpu_weights(c)
    X, am, fm = bf16(c["X"]), u8(c["attn_mask"]), u8(c["ffn_mask"])
    kw = dict(n_q=nq, n_kv=nkv, rope_theta=m["rope_theta"], eps=m["eps"])
    if entry == "layer_masked_cache":
        K, V = bf16(c["K_cache"]), bf16(c["V_cache"])
        lens = i32(np.random.default_rng(6).integers(0, L + 1, size=(B, nkv)))
        fn = lambda out: wide.layer_decode_masked_cache(X, am, fm, Wl, K_cache=K, V_cache=V,
                                                        kv_len=lens, pos=L, out=out, **kw)
        caches = [K, V]
    else:
        p = paged_cache(f"graph_{entry}", B, nkv, 16, 20)
        Kp, Vp = bf16(p["K_pool"]), bf16(p["V_pool"])
        tab, pl = i32(p["page_table"]), i32(p["kv_len"])
        fn = lambda out: wide.layer_decode_masked_paged(X, am, fm, Wl, K_pool=Kp, V_pool=Vp,
                                                        page_table=tab, kv_len=pl, pos=319,
                                                        out=out, **kw)
        caches = [Kp, Vp]
    _replays_match((B, d), fn, caches)
