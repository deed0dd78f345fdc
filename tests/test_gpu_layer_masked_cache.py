"""GPU parity of the whole layer decoding over masked K/V caches (reading R5 carried
across steps): wide_layer_decode_masked_cache (per-(sequence, group) lengths) and
wide_layer_decode_masked_paged (the same caches in pages of a pool).

A layer decode run token by token from empty caches, advancing each pair's length by
the attention mask, must reproduce the oracle's prefill rows of the same tokens; the
paged run must equal the contiguous run bit for bit.  One step with lengths spread
over the whole range is checked at the Llama-3.1-8B decode shape."""
import zlib

import numpy as np
import torch

import sparse_wide_mask_amd as wide
from oracle import layer_masked
from synth.workloads import layer_8b, layer_case
from tests._gpu import TOL, bf16, dev, host, log, nan_bf16, needs_gpu, rel_err, u8
from tests.test_gpu_layer import gpu_weights


def _oracle_prefill(c, X, am, fm):
    m = c["meta"]
    return layer_masked(X, am, fm, c, n_q=m["n_q"], n_kv=m["n_kv"], head_dim=128,
                        n_ffn=m["n_ffn"], rope_theta=m["rope_theta"], eps=m["eps"])


@needs_gpu
def test_layer_masked_cache_steps_reproduce_prefill():
    """20 layer decode steps of 4 sequences from empty caches (contiguous, and paged
    with pages of 16 slots taken from a shuffled free list): every step's output
    equals the oracle's prefill row of that token, and paged equals contiguous."""
    dev()
    log("layer masked-cache decode, 20 steps vs prefill (contiguous and paged)")
    B, S, d, F, n_ffn, n_q, n_kv, ps = 4, 20, 256, 1024, 8, 8, 2, 16
    seqs = [layer_case(f"lmc_seq_{b}", S, d, F, n_ffn, n_q, n_kv, 128, 0.5, "bernoulli")
            for b in range(B)]
    c = seqs[0]
    m = c["meta"]
    W = gpu_weights(c)
    X = np.stack([s["X"] for s in seqs])
    AM = np.stack([s["attn_mask"] for s in seqs])
    FM = np.stack([s["ffn_mask"] for s in seqs])
    Kc = torch.zeros((B, n_kv, S, 128), dtype=torch.bfloat16, device=dev())
    Vc = torch.zeros_like(Kc)
    max_pages = (S + ps - 1) // ps
    n_pages = B * n_kv * max_pages + 3
    free = list(np.random.default_rng(11).permutation(n_pages))
    table = np.full((B, n_kv, max_pages), -1, np.int32)
    Kp = torch.zeros((n_pages, ps, 128), dtype=torch.bfloat16, device=dev())
    Vp = torch.zeros_like(Kp)
    L = np.zeros((B, n_kv), np.int32)
    got, got_paged = [], []
    kw = dict(n_q=n_q, n_kv=n_kv, rope_theta=m["rope_theta"], eps=m["eps"])
    for s in range(S):
        for b, g in zip(*np.nonzero(AM[:, s])):
            if L[b, g] % ps == 0:            # the new slot opens a page
                table[b, g, L[b, g] // ps] = free.pop()
        x, am, fm = bf16(np.ascontiguousarray(X[:, s])), u8(AM[:, s]), u8(FM[:, s])
        Ld = torch.from_numpy(L).to(dev())
        got.append(host(wide.layer_decode_masked_cache(
            x, am, fm, W, K_cache=Kc, V_cache=Vc, kv_len=Ld, pos=s, out=nan_bf16((B, d)), **kw)))
        got_paged.append(host(wide.layer_decode_masked_paged(
            x, am, fm, W, K_pool=Kp, V_pool=Vp, page_table=torch.from_numpy(table).to(dev()),
            kv_len=Ld, pos=s, out=nan_bf16((B, d)), **kw)))
        L += (AM[:, s] != 0).astype(np.int32)
    torch.cuda.synchronize()
    for b in range(B):
        ref = _oracle_prefill(c, X[b], AM[b], FM[b])
        mine = np.stack([g[b] for g in got])
        assert rel_err(mine, ref) <= TOL
        assert np.array_equal(mine, np.stack([g[b] for g in got_paged])), "paged != contiguous"


@needs_gpu
def test_layer_masked_cache_llama31_8b():
    """Llama-3.1-8B layer decode, batch 32, caches of 8193 slots with per-pair lengths
    spread over the whole range (new token at position 8192): output, the appended
    K/V and the untouched slots against the oracle."""
    dev()
    log("layer masked-cache decode 8B B=32 cap=8193")
    c = layer_8b(32, decode=True, L=8192)
    m = c["meta"]
    B, n_kv, cap = 32, 8, c["K_cache"].shape[2]
    rng = np.random.default_rng(zlib.crc32(b"lmc_8b"))
    L = rng.integers(0, cap, size=(B, n_kv)).astype(np.int32)
    L.flat[0], L.flat[-1] = 0, cap - 1
    Kc, Vc = bf16(c["K_cache"]), bf16(c["V_cache"])
    Y = wide.layer_decode_masked_cache(bf16(c["X"]), u8(c["attn_mask"]), u8(c["ffn_mask"]),
                                       gpu_weights(c), n_q=32, n_kv=8, K_cache=Kc, V_cache=Vc,
                                       kv_len=torch.from_numpy(L).to(dev()), pos=8192,
                                       rope_theta=m["rope_theta"], eps=m["eps"],
                                       out=nan_bf16((B, 4096)))
    torch.cuda.synchronize()
    ref, parts = layer_masked(c["X"], c["attn_mask"], c["ffn_mask"], c, n_q=32, n_kv=8,
                              head_dim=128, n_ffn=112, rope_theta=m["rope_theta"], eps=m["eps"],
                              decode=True, K_cache=c["K_cache"], V_cache=c["V_cache"], kv_len=L,
                              pos=8192, return_parts=True)
    assert rel_err(host(Y), ref) <= TOL
    delta = parts["a"] + parts["f"]
    bound = TOL * np.abs(delta).max() + 2.0 ** -8 * (np.abs(parts["h"]).max() + np.abs(ref).max())
    assert np.abs((host(Y) - c["X"]) - delta).max() <= bound
    Kg, Vg = host(Kc), host(Vc)
    K0, V0 = c["K_cache"].copy(), c["V_cache"].copy()
    for b, g in zip(*np.nonzero(c["attn_mask"])):
        assert rel_err(Kg[b, g, L[b, g]], parts["K_new"][b, g]) <= TOL
        K0[b, g, L[b, g]] = Kg[b, g, L[b, g]]
        V0[b, g, L[b, g]] = Vg[b, g, L[b, g]]
    assert np.array_equal(Kg, K0) and np.array_equal(Vg, V0), "cache written outside kept slots"
