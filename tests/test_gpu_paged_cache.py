"""GPU parity of wide_attn_decode_masked_paged: the masked-cache decode over a
paged cache (pools of pages and a page table per (sequence, group)).

The oracle gathers the pages into contiguous caches (reading R10) and runs the
per-pair decode (R5).  The outputs and the new rows match it to the bf16
tolerance; every other pool row is unchanged bit for bit.  With the same logical
caches, the paged call's output equals the contiguous masked-cache call's bit for
bit (the same arithmetic, only the addresses differ)."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import attn_masked, paged_to_contiguous
from synth.workloads import attn_case, paged_cache
from tests._gpu import TOL, bf16, dev, host, log, nan_bf16, needs_gpu, rel_err, u8


def _weights(c):
    m = c["meta"]
    return (bf16(c["Wq"]), bf16(c["Wk"]), bf16(c["Wv"]), wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]))


def _gpu_paged(c, p, pos, theta, W=None):
    m = c["meta"]
    B, d = c["X"].shape
    Kp, Vp = bf16(p["K_pool"]), bf16(p["V_pool"])
    Y = nan_bf16((B, d))
    wide.attn_decode_masked_paged(bf16(c["X"]), u8(c["mask"]), *(W or _weights(c)), n_q=m["n_q"],
                                  n_kv=m["n_kv"], K_pool=Kp, V_pool=Vp,
                                  page_table=torch.from_numpy(p["page_table"]).to(dev()),
                                  kv_len=torch.from_numpy(p["kv_len"]).to(dev()), pos=pos,
                                  rope_theta=theta, out=Y)
    torch.cuda.synchronize()
    return host(Y), host(Kp), host(Vp)


def _check(c, p, pos, theta, contiguous_too=True):
    m = c["meta"]
    B, d = c["X"].shape
    W = _weights(c)
    Y, Kg, Vg = _gpu_paged(c, p, pos, theta, W)
    Kc, Vc, Le = paged_to_contiguous(p["K_pool"], p["V_pool"], p["page_table"], p["kv_len"])
    Yr, Kn, Vn = attn_masked(c["X"], c["mask"], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                             n_kv=m["n_kv"], head_dim=128, rope_theta=theta, decode=True,
                             K_cache=Kc, V_cache=Vc, kv_len=Le, pos=pos)
    assert rel_err(Y, Yr) <= TOL
    ps, table = p["K_pool"].shape[1], p["page_table"]
    K0, V0 = p["K_pool"].copy(), p["V_pool"].copy()
    cap = Kc.shape[2]
    for b, g in zip(*np.nonzero((c["mask"] != 0) & (Le >= 0) & (Le < cap))):
        page, row = table[b, g, Le[b, g] // ps], Le[b, g] % ps
        assert rel_err(Kg[page, row], Kn[b, g]) <= TOL
        assert rel_err(Vg[page, row], Vn[b, g]) <= TOL
        K0[page, row], V0[page, row] = Kg[page, row], Vg[page, row]
    assert np.array_equal(Kg, K0) and np.array_equal(Vg, V0), "pool written outside new slots"
    if contiguous_too:
        # the contiguous call on the gathered caches: the same output, bit for bit
        Yc = nan_bf16((B, d))
        wide.attn_decode_masked_cache(bf16(c["X"]), u8(c["mask"]), *W, n_q=m["n_q"],
                                      n_kv=m["n_kv"], K_cache=bf16(Kc), V_cache=bf16(Vc),
                                      kv_len=torch.from_numpy(Le.astype(np.int32)).to(dev()),
                                      pos=pos, rope_theta=theta, out=Yc)
        torch.cuda.synchronize()
        assert np.array_equal(host(Yc), Y), "paged and contiguous outputs differ"


CASES = [
    # B, d, n_q, n_kv, page_size, max_pages, pos, keep, kind, theta, unmapped
    (3, 256, 8, 2, 16, 3, 47, 0.5, "bernoulli", 500000.0, 0.0),
    (16, 256, 32, 8, 16, 20, 400, 0.5, "topk", 0.0, 0.0),        # chunks over 8 pages
    (40, 320, 8, 2, 64, 5, 319, 0.5, "topk", 500000.0, 0.0),      # batch over 16
    (64, 512, 16, 4, 128, 3, 1000, 0.75, "clustered", 10000.0, 0.0),
    (7, 384, 12, 4, 256, 3, 767, 0.5, "bernoulli", 500000.0, 0.0),  # r = 3, chunk in a page
    (5, 256, 16, 4, 1024, 1, 5, 1.0, "ones", 0.0, 0.0),            # one page per pair
    (9, 256, 8, 2, 32, 12, 383, 0.75, "topk", 500000.0, 0.3),     # unmapped entries
    (24, 256, 16, 16, 32, 6, 191, 0.5, "bernoulli", 500000.0, 0.0),  # r = 1, 16 groups
]


@needs_gpu
@pytest.mark.parametrize("B,d,n_q,n_kv,ps,max_pages,pos,keep,kind,theta,unmapped", CASES)
def test_paged_cache_shapes(B, d, n_q, n_kv, ps, max_pages, pos, keep, kind, theta, unmapped):
    dev()
    log(f"paged decode B={B} d={d} n_q={n_q} n_kv={n_kv} page={ps}x{max_pages} pos={pos} {kind} "
        f"unmapped={unmapped}")
    c = attn_case(f"paged_{B}_{ps}_{kind}", B, d, n_q, n_kv, 128, keep, kind)
    p = paged_cache(f"paged_{B}_{ps}_{max_pages}", B, n_kv, ps, max_pages, unmapped=unmapped)
    _check(c, p, pos, theta)


@needs_gpu
def test_paged_cache_unmapped_new_slots_and_bad_lengths():
    """Pairs whose new slot is on an unmapped page (entry -1 or past the pool) and
    pairs with lengths outside the capacity behave like dropped pairs: zero output
    for their heads, nothing written."""
    dev()
    log("paged decode, unmapped new slots and out-of-range lengths")
    B, d, n_q, n_kv, ps, max_pages = 6, 256, 8, 2, 16, 4
    c = attn_case("paged_bad", B, d, n_q, n_kv, 128, 1.0, "ones")
    p = paged_cache("paged_bad", B, n_kv, ps, max_pages)
    t, L = p["page_table"], p["kv_len"]
    L[0, 0], t[0, 0, 40 // ps] = 40, -1                 # new slot on an unmapped page (-1)
    L[1, 1], t[1, 1, 17 // ps] = 17, p["meta"]["n_pages"]  # ... on an entry past the pool
    L[2, 0], L[3, 1] = -1, max_pages * ps                # lengths outside the capacity
    _check(c, p, 63, 500000.0)
    # the same call with those four pairs dropped by the mask instead: the same
    # output bit for bit (both feed zeros for those heads into the O projection)
    Y, _, _ = _gpu_paged(c, p, 63, 500000.0)
    c2 = dict(c, mask=c["mask"].copy())
    for b, g in ((0, 0), (1, 1), (2, 0), (3, 1)):
        c2["mask"][b, g] = 0
    Y2, _, _ = _gpu_paged(c2, p, 63, 500000.0)
    assert np.array_equal(Y, Y2)


@needs_gpu
def test_paged_cache_shared_prefix_pages():
    """Every (sequence, group) reads the same first 3 pages (a shared prefix) and
    appends past them into pages of its own."""
    dev()
    log("paged decode, shared prefix pages")
    B, d, n_q, n_kv = 12, 256, 16, 4
    c = attn_case("paged_shared", B, d, n_q, n_kv, 128, 0.5, "topk")
    p = paged_cache("paged_shared", B, n_kv, 32, 8, shared_pages=3)
    _check(c, p, 255, 500000.0)


@needs_gpu
def test_paged_cache_steps_reproduce_prefill():
    """20 decode steps from an empty pool, pages of 16 slots taken from a free list
    in shuffled order as each (sequence, group) fills its last one: every step's
    output equals the oracle's prefill row of that token."""
    dev()
    log("paged decode, 20 steps vs prefill")
    B, S, d, n_q, n_kv, ps, theta = 4, 20, 256, 8, 2, 16, 500000.0
    seqs = [attn_case(f"paged_seq_{b}", S, d, n_q, n_kv, 128, 0.6, "bernoulli") for b in range(B)]
    W = seqs[0]
    X = np.stack([s["X"] for s in seqs])
    M = np.stack([s["mask"] for s in seqs])
    Wt = _weights(W)
    max_pages = (S + ps - 1) // ps
    n_pages = B * n_kv * max_pages + 2
    free = list(np.random.default_rng(3).permutation(n_pages))
    table = np.full((B, n_kv, max_pages), -1, np.int32)
    Kp = torch.zeros((n_pages, ps, 128), dtype=torch.bfloat16, device=dev())
    Vp = torch.zeros_like(Kp)
    L = np.zeros((B, n_kv), np.int32)
    got = []
    for s in range(S):
        for b, g in zip(*np.nonzero(M[:, s])):
            if L[b, g] % ps == 0:            # the new slot opens a page
                table[b, g, L[b, g] // ps] = free.pop()
        got.append(host(wide.attn_decode_masked_paged(
            bf16(np.ascontiguousarray(X[:, s])), u8(M[:, s]), *Wt, n_q=n_q, n_kv=n_kv,
            K_pool=Kp, V_pool=Vp, page_table=torch.from_numpy(table).to(dev()),
            kv_len=torch.from_numpy(L).to(dev()), pos=s, rope_theta=theta)))
        L += (M[:, s] != 0).astype(np.int32)
    for b in range(B):
        ref = attn_masked(X[b], M[b], W["Wq"], W["Wk"], W["Wv"], W["Wo"], n_q=n_q, n_kv=n_kv,
                          head_dim=128, rope_theta=theta)
        assert rel_err(np.stack([g[b] for g in got]), ref) <= TOL


@needs_gpu
def test_paged_cache_llama31_8b():
    """Llama-3.1-8B attention decode shape: batch 16, pages of 16 slots, 257 pages a
    pair (4112 slots), lengths over the whole range, keep 4 of 8."""
    dev()
    log("paged decode 8B B=16 page=16x257")
    c = attn_case("paged_8b", 16, 4096, 32, 8, 128, 0.5, "topk")
    p = paged_cache("paged_8b", 16, 8, 16, 257)
    _check(c, p, 4111, 500000.0)
