"""GPU parity of wide_router_topk against the oracle (reading R9).

The logits are floating point: within 1e-3 of the fp64 oracle (bf16 inputs,
fp32 accumulation).  The selection is an integer decision taken on floating
point, so both sides take it on the same numbers: the oracle selects on the
logits the GPU returned, and the mask and packed words must match bit for bit.
At full size the oracle (quadratic loops) checks sampled tokens; every row is
checked for properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
import synth
from oracle import router_topk
from tests._gpu import bf16, dev, host, log, needs_gpu, rel_err

LOGIT_TOL = 1e-3


def _inputs(tag, T, d, n):
    X = synth.normal(f"router_{tag}", "X", (T, d))
    R = synth.normal(f"router_{tag}", "R", (n, d), std=d ** -0.5)
    return X, R


def _packed_of(mask):
    T, n = mask.shape
    nw = (n + 63) // 64
    pad = np.zeros((T, nw * 64), np.uint8)
    pad[:, :n] = mask
    return np.packbits(pad, axis=1, bitorder="little").view("<u8").reshape(T, nw)


def _check_rows(L, mask, k):
    """Every row keeps exactly k groups, each ranking before every dropped one."""
    assert np.all(mask.sum(axis=1) == k)
    if 0 < k < L.shape[1]:
        kept_min = np.where(mask == 1, L, np.inf).min(axis=1)
        drop_max = np.where(mask == 0, L, -np.inf).max(axis=1)
        assert np.all(kept_min >= drop_max)
        # at equal values the kept ones have the lower group indices
        for t in np.flatnonzero(kept_min == drop_max):
            v = kept_min[t]
            eq = np.flatnonzero(L[t] == v)
            kept_eq = eq[mask[t, eq] == 1]
            drop_eq = eq[mask[t, eq] == 0]
            assert kept_eq.max() < drop_eq.min()


def _run(X, R, k, rows=None):
    Xd, Rp = bf16(X), wide.pack_router(bf16(R))
    n = R.shape[0]
    out = wide.router_topk(Xd, Rp, k, n, return_logits=True)
    bare = wide.router_topk(Xd, Rp, k, n)  # no logits requested: the same selection
    torch.cuda.synchronize()
    L = host(out["logits"]).astype(np.float64)
    mask = host(out["mask"])
    packed = host(out["packed"]).view(np.uint64)
    assert np.array_equal(host(bare["mask"]), mask)
    assert np.array_equal(host(bare["packed"]).view(np.uint64), packed)
    sel = slice(None) if rows is None else rows
    ref = router_topk(X[sel], R, k)
    assert rel_err(L[sel], ref["logits"]) <= LOGIT_TOL
    on_gpu_logits = router_topk(None, None, k, logits=L[sel])
    np.testing.assert_array_equal(mask[sel], on_gpu_logits["mask"])
    np.testing.assert_array_equal(packed[sel], on_gpu_logits["packed"])
    np.testing.assert_array_equal(packed, _packed_of(mask))
    _check_rows(L, mask, k)
    return L, mask


SHAPES = [
    (1, 64, 1, 1), (5, 64, 3, 2), (33, 128, 16, 8), (100, 256, 112, 56), (64, 256, 256, 100),
    (70, 192, 10, 3), (300, 3072, 64, 32), (40, 512, 8, 0), (40, 512, 8, 8), (17, 320, 130, 65),
    (257, 4096, 8, 4),
]


@needs_gpu
@pytest.mark.parametrize("T,d,n,k", SHAPES)
def test_router_shapes(T, d, n, k):
    dev()
    log(f"router T={T} d={d} n={n} k={k}")
    X, R = _inputs(f"{T}_{d}_{n}", T, d, n)
    _run(X, R, k)


@needs_gpu
def test_router_ties_go_to_the_lower_group():
    dev()
    log("router ties")
    T, d, n, k = 50, 128, 20, 7
    X, R = _inputs("ties", T, d, n)
    R[1::2] = R[0::2]                       # groups 2i and 2i+1 get equal logits
    X[:10] = 0.0                            # rows of zeros: every logit is +-0
    L, mask = _run(X, R, k)
    np.testing.assert_array_equal(mask[:10], np.tile((np.arange(n) < k).astype(np.uint8), (10, 1)))
    assert np.all(L[10:, 0::2] == L[10:, 1::2])


@needs_gpu
@pytest.mark.parametrize("n,k", [(112, 56), (8, 4)])
def test_router_llama31_8b_full(n, k):
    """The layer's router shapes: 8192 tokens of d_model 4096, 112 FFN groups keeping
    56 and 8 head groups keeping 4; the oracle checks 64 sampled tokens, properties
    every token."""
    dev()
    log(f"router full n={n} k={k}")
    X, R = _inputs(f"full_{n}", 8192, 4096, n)
    rows = np.random.default_rng(n).choice(8192, 64, replace=False)
    _run(X, R, k, rows=np.sort(rows))


@needs_gpu
@pytest.mark.parametrize("n,d", [(112, 4096), (8, 256), (130, 320), (1, 64)])
def test_pack_router_is_the_fragment_order(n, d):
    """Block (j, s), row l of the packed weights is R[16 j + l % 16, 32 s + 8 (l // 16) :+8],
    zeros past n; checked bit for bit against a NumPy rearrangement."""
    dev()
    _, R = _inputs(f"pack_{n}_{d}", 1, d, n)
    got = host(wide.pack_router(bf16(R))).reshape(-1)
    nt, ns = (n + 15) // 16, d // 32
    Rpad = np.zeros((nt * 16, d), np.float32)
    Rpad[:n] = R
    ref = Rpad.reshape(nt, 16, ns, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    np.testing.assert_array_equal(got, ref)
