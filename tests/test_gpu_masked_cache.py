"""GPU parity of wide_attn_decode_masked_cache: decode over caches in which tokens
that skipped a group left no entry, so every (sequence, group) has its own length.

The outputs and the new cache slots are compared with the oracle (reading R5 with
per-pair lengths) to the bf16 tolerance; every other cache slot must be unchanged
bit for bit.  A decode run token by token from empty caches must reproduce the
oracle's prefill rows (reading R4 carried across steps)."""
import zlib

import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import attn_masked
from synth.workloads import attn_case
from tests._gpu import TOL, bf16, dev, host, log, nan_bf16, needs_gpu, rel_err, u8


def _lengths(tag, B, n_kv, cap):
    rng = np.random.default_rng(zlib.crc32(tag.encode()))
    L = rng.integers(0, cap, size=(B, n_kv)).astype(np.int32)
    L.flat[0] = 0
    L.flat[-1] = cap - 1
    return L


def _gpu(c, L, pos, theta):
    m = c["meta"]
    B, d = c["X"].shape
    Kc, Vc = bf16(c["K_cache"]), bf16(c["V_cache"])
    Y = nan_bf16((B, d))
    wide.attn_decode_masked_cache(bf16(c["X"]), u8(c["mask"]), bf16(c["Wq"]), bf16(c["Wk"]),
                                  bf16(c["Wv"]), wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]),
                                  n_q=m["n_q"], n_kv=m["n_kv"], K_cache=Kc, V_cache=Vc,
                                  kv_len=torch.from_numpy(L).to(dev()), pos=pos, rope_theta=theta,
                                  out=Y)
    torch.cuda.synchronize()
    return host(Y), host(Kc), host(Vc)


def _check(c, L, pos, theta):
    m = c["meta"]
    Y, Kg, Vg = _gpu(c, L, pos, theta)
    Yr, Kn, Vn = attn_masked(c["X"], c["mask"], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                             n_kv=m["n_kv"], head_dim=128, rope_theta=theta, decode=True,
                             K_cache=c["K_cache"], V_cache=c["V_cache"], kv_len=L, pos=pos)
    assert rel_err(Y, Yr) <= TOL
    cap = c["K_cache"].shape[2]
    K0, V0 = c["K_cache"].copy(), c["V_cache"].copy()
    for b, g in zip(*np.nonzero((c["mask"] != 0) & (L >= 0) & (L < cap))):
        # the new token's k/v at slot kv_len[b, g] of the kept pairs only
        assert rel_err(Kg[b, g, L[b, g]], Kn[b, g]) <= TOL
        assert rel_err(Vg[b, g, L[b, g]], Vn[b, g]) <= TOL
        K0[b, g, L[b, g]] = Kg[b, g, L[b, g]]
        V0[b, g, L[b, g]] = Vg[b, g, L[b, g]]
    assert np.array_equal(Kg, K0) and np.array_equal(Vg, V0), "cache written outside kept slots"


CASES = [
    # B, d, n_q, n_kv, cap, pos, keep, kind, theta
    (3, 256, 8, 2, 40, 39, 0.5, "bernoulli", 500000.0),
    (16, 256, 32, 8, 300, 512, 0.5, "topk", 0.0),
    (40, 320, 8, 2, 131, 130, 0.5, "topk", 500000.0),     # batch over 16: LDS-shared rows
    (64, 512, 16, 4, 260, 1000, 0.75, "clustered", 10000.0),
    (5, 256, 16, 4, 1, 0, 1.0, "ones", 0.0),              # one slot: every length is 0
    (7, 384, 12, 4, 700, 699, 0.5, "bernoulli", 500000.0),  # r = 3
    (40, 256, 16, 16, 150, 149, 0.5, "topk", 500000.0),     # r = 1, 16 groups
    (2, 256, 8, 2, 17000, 16999, 0.5, "bernoulli", 500000.0),  # over 128 chunks a pair
]


@needs_gpu
@pytest.mark.parametrize("B,d,n_q,n_kv,cap,pos,keep,kind,theta", CASES)
def test_masked_cache_shapes(B, d, n_q, n_kv, cap, pos, keep, kind, theta):
    dev()
    log(f"masked-cache decode B={B} d={d} n_q={n_q} n_kv={n_kv} cap={cap} pos={pos} {kind}")
    c = attn_case(f"mcache_{B}_{cap}_{kind}", B, d, n_q, n_kv, 128, keep, kind, decode=True,
                  kv_len=cap - 1, kv_cap=cap)
    _check(c, _lengths(f"{B}_{cap}", B, n_kv, cap), pos, theta)


@needs_gpu
def test_masked_cache_out_of_range_lengths():
    """Lengths outside [0, kv_cap) behave like dropped pairs: no write, zero output."""
    dev()
    log("masked-cache decode, out-of-range lengths")
    B, d, n_q, n_kv, cap = 6, 256, 8, 2, 50
    c = attn_case("mcache_bad", B, d, n_q, n_kv, 128, 1.0, "ones", decode=True,
                  kv_len=cap - 1, kv_cap=cap)
    L = _lengths("bad", B, n_kv, cap)
    L[0, 0], L[1, 1], L[2, 0] = -1, cap, 2 ** 30
    _check(c, L, 77, 500000.0)


@needs_gpu
def test_masked_cache_steps_reproduce_prefill():
    """24 decode steps from empty caches, advancing each pair's length by its mask:
    every step's output equals the oracle's prefill row of that token."""
    dev()
    log("masked-cache decode, 24 steps vs prefill")
    B, S, d, n_q, n_kv, theta = 4, 24, 256, 8, 2, 500000.0
    seqs = [attn_case(f"mcache_seq_{b}", S, d, n_q, n_kv, 128, 0.5, "bernoulli") for b in range(B)]
    W = seqs[0]
    X = np.stack([s["X"] for s in seqs])                 # [B, S, d]
    M = np.stack([s["mask"] for s in seqs])              # [B, S, n_kv]
    Wq, Wk, Wv = bf16(W["Wq"]), bf16(W["Wk"]), bf16(W["Wv"])
    Wo = wide.pack_kmajor(bf16(W["Wo"]), n_kv)
    Kc = torch.zeros((B, n_kv, S, 128), dtype=torch.bfloat16, device=dev())
    Vc = torch.zeros_like(Kc)
    L = torch.zeros((B, n_kv), dtype=torch.int32, device=dev())
    got = []
    for s in range(S):
        mask = u8(M[:, s])
        got.append(host(wide.attn_decode_masked_cache(bf16(np.ascontiguousarray(X[:, s])), mask,
                                                      Wq, Wk, Wv, Wo, n_q=n_q, n_kv=n_kv,
                                                      K_cache=Kc, V_cache=Vc, kv_len=L, pos=s,
                                                      rope_theta=theta)))
        L += (mask != 0).to(torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(L), M.sum(axis=1))
    for b in range(B):
        ref = attn_masked(X[b], M[b], W["Wq"], W["Wk"], W["Wv"], W["Wo"], n_q=n_q, n_kv=n_kv,
                          head_dim=128, rope_theta=theta)
        assert rel_err(np.stack([g[b] for g in got]), ref) <= TOL


@needs_gpu
def test_masked_cache_llama31_8b():
    """Llama-3.1-8B attention decode shape: batch 16, caches of 4097 slots holding
    per-pair lengths across the whole range, keep 4 of 8."""
    dev()
    log("masked-cache decode 8B B=16 cap=4097")
    c = attn_case("mcache_8b", 16, 4096, 32, 8, 128, 0.5, "topk", decode=True, kv_len=4096,
                  kv_cap=4097)
    _check(c, _lengths("8b", 16, 8, 4097), 4096, 500000.0)
