"""A layer call recorded into a HIP graph (torch.cuda.graph) replays to the eager
result bit for bit.  Prefill forks the mask reorders onto the library's second
stream and joins them back with events, which capture turns into graph edges;
decode appends to the caches at the same slot on every replay.  Each replay is
preceded by eager work on the same buffers (a fill of the output, an eager call
into another output) and checked on its own."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from synth.workloads import layer_case
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
