"""Pins of the oracle's mask reordering (gist.science technical summary §2.B).

The oracle builds every output with explicit loops.  Here each output is checked
against a library routine that computes the same object a different way
(np.argsort stable, np.packbits, np.any), against invariants, against a
hand-worked fixture and by brute force over every mask of tiny shapes.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import mask_reorder

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lib_reference(m, tile_m):
    m = (np.asarray(m) != 0).astype(np.uint8)
    T, n = m.shape
    nw = (n + 63) // 64
    pad = np.zeros((T, nw * 64), np.uint8)
    pad[:, :n] = m
    packed = np.packbits(pad, axis=1, bitorder="little").view("<u8").reshape(T, nw)
    perm = np.stack([np.argsort(1 - m[:, g], kind="stable") for g in range(n)]) if n else np.zeros((0, T))
    rank = np.argsort(perm, axis=1) if n else perm
    count = m.sum(axis=0)
    nt = -(-T // tile_m)
    tg = np.full((nt, n), -1)
    tc = np.zeros(nt, int)
    for i in range(nt):
        any_ = np.any(m[i * tile_m:(i + 1) * tile_m], axis=0)
        idx = np.flatnonzero(any_)
        tg[i, :idx.size] = idx
        tc[i] = idx.size
    return dict(packed=packed, group_count=count, group_perm=perm, group_rank=rank,
                tile_count=tc, tile_groups=tg)


def _check_equal(out, ref):
    for k in ref:
        np.testing.assert_array_equal(np.asarray(out[k]).astype(np.int64),
                                      np.asarray(ref[k]).astype(np.int64), err_msg=k)


def _check_invariants(m, out):
    m = np.asarray(m) != 0
    T, n = m.shape
    perm, rank, cnt = out["group_perm"], out["group_rank"], out["group_count"]
    for g in range(n):
        assert sorted(perm[g].tolist()) == list(range(T))
        np.testing.assert_array_equal(rank[g][perm[g]], np.arange(T))
        np.testing.assert_array_equal(m[perm[g], g], np.arange(T) < cnt[g])
        a = perm[g][:cnt[g]]
        assert np.all(np.diff(a) > 0) and np.all(np.diff(perm[g][cnt[g]:]) > 0)
    assert cnt.sum() == m.sum()


def test_golden_hand_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "reorder_6x3.json")))
    out = mask_reorder(np.array(fx["mask"], np.uint8), fx["tile_m"])
    for k in ("packed", "group_count", "group_perm", "group_rank", "tile_count", "tile_groups"):
        np.testing.assert_array_equal(np.asarray(out[k]).astype(np.int64), np.array(fx[k]), err_msg=k)


@pytest.mark.parametrize("T,n,tile_m", [(1, 1, 1), (5, 3, 2), (63, 8, 64), (64, 64, 64),
                                         (65, 65, 64), (130, 112, 128), (200, 63, 7),
                                         (97, 129, 33)])
@pytest.mark.parametrize("p", [0.0, 0.3, 0.5, 1.0])
def test_against_library(T, n, tile_m, p):
    rng = np.random.default_rng(T * 1000 + n + int(p * 10))
    m = (rng.random((T, n)) < p).astype(np.uint8) * rng.integers(1, 256, (T, n)).astype(np.uint8)
    out = mask_reorder(m, tile_m)
    _check_equal(out, _lib_reference(m, tile_m))
    _check_invariants(m, out)


@pytest.mark.parametrize("T,n", [(3, 4), (4, 3), (2, 6), (6, 2), (12, 1)])
def test_brute_force_all_masks(T, n):
    """Every one of the 2^(T*n) masks, against Python's sorted() with key (dropped, t)."""
    for bits in itertools.product((0, 1), repeat=T * n):
        m = np.array(bits, np.uint8).reshape(T, n)
        out = mask_reorder(m, 2)
        for g in range(n):
            order = sorted(range(T), key=lambda t: (m[t, g] == 0, t))
            assert out["group_perm"][g].tolist() == order
            assert out["group_count"][g] == sum(m[:, g])
        for i in range(-(-T // 2)):
            kept = sorted({g for t in range(2 * i, min(T, 2 * i + 2)) for g in range(n) if m[t, g]})
            assert out["tile_count"][i] == len(kept)
            assert out["tile_groups"][i][:len(kept)].tolist() == kept
            assert all(v == -1 for v in out["tile_groups"][i][len(kept):])
        w = [sum(int(m[t, g]) << g for g in range(n)) for t in range(T)]
        assert out["packed"][:, 0].tolist() == w
