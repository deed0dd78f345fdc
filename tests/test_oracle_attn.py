"""Pins of the oracle's masked attention sublayer (gist.science §2.A GQA-aligned
head groups; readings R3-R5).

Against torch SDPA and transformers' Llama rotary embedding (float64, CPU):
all-ones = dense causal GQA; for every group the kept rows equal dense causal
attention over the group's kept tokens at their original positions; a group's
first kept token gets its own value row; skipped groups give exact zeros; decode
against SDPA over cache + new token, and decode = last row of prefill.
"""
import itertools

import numpy as np
import pytest

from oracle import attn_masked, rope
from tests._libref import qkv_lib, rope_lib, sdpa, t64


def _rope_tol(pos, x):
    """Bound for results that pass through transformers' float32 rotary tables."""
    return 4.0 * float(np.max(pos) + 1) * 2.0 ** -23 * float(np.max(np.abs(x)) + 1)


def _tol(theta, T):
    return 1e-11 if not theta else 50.0 * T * 2.0 ** -23


def _w(d, n_q, n_kv, hd, seed, s=0.3):
    r = np.random.default_rng(seed)
    return dict(Wq=r.standard_normal((n_q * hd, d)) * s, Wk=r.standard_normal((n_kv * hd, d)) * s,
                Wv=r.standard_normal((n_kv * hd, d)) * s, Wo=r.standard_normal((n_q * hd, d)) * s)


def _run(X, m, W, n_q, n_kv, hd, theta, **kw):
    return attn_masked(X, m, W["Wq"], W["Wk"], W["Wv"], W["Wo"], n_q=n_q, n_kv=n_kv,
                       head_dim=hd, rope_theta=theta, **kw)


# ----------------------------------------------------------------- RoPE

@pytest.mark.parametrize("theta", [10000.0, 500000.0])
def test_rope_matches_transformers(theta):
    x = np.random.default_rng(0).standard_normal((37, 3, 16))
    pos = np.arange(37) * 7 + 3
    # transformers builds inv_freq and pos*inv_freq in float32: its angles carry an
    # error of about max(pos) * 2^-23, which bounds the difference here.
    np.testing.assert_allclose(rope(x, pos, theta), rope_lib(x, pos, theta), rtol=0,
                               atol=_rope_tol(pos, x))


def test_rope_properties():
    r = np.random.default_rng(1)
    x = r.standard_normal((1, 1, 32))
    np.testing.assert_array_equal(rope(x, [0], 500000.0), x)           # pos 0 = identity
    pos = np.arange(50) * 131
    xs = np.repeat(x, 50, axis=0)
    y = rope(xs, pos, 500000.0)
    half = 16
    pn_in = xs[..., :half] ** 2 + xs[..., half:] ** 2
    pn_out = y[..., :half] ** 2 + y[..., half:] ** 2
    np.testing.assert_allclose(pn_out, pn_in, rtol=1e-12)              # each pair keeps its norm
    q, k = r.standard_normal(32), r.standard_normal(32)
    d1 = rope(q[None, None], [1000], 500000.0).ravel() @ rope(k[None, None], [990], 500000.0).ravel()
    d2 = rope(q[None, None], [20], 500000.0).ravel() @ rope(k[None, None], [10], 500000.0).ravel()
    assert abs(d1 - d2) < 1e-10                                          # depends only on t - s


# ---------------------------------------------------------------- prefill

@pytest.mark.parametrize("theta", [0.0, 500000.0])
@pytest.mark.parametrize("n_q,n_kv", [(4, 2), (8, 2), (4, 4)])
def test_all_ones_is_causal_gqa(theta, n_q, n_kv):
    T, d, hd = 23, 32, 8
    W = _w(d, n_q, n_kv, hd, 2)
    X = np.random.default_rng(3).standard_normal((T, d))
    Y = _run(X, np.ones((T, n_kv), np.uint8), W, n_q, n_kv, hd, theta)
    q, k, v = qkv_lib(X, W["Wq"], W["Wk"], W["Wv"], n_q, n_kv, hd, theta, np.arange(T))
    o = sdpa(q, k, v, causal=True).reshape(T, n_q * hd)
    np.testing.assert_allclose(Y, (t64(o) @ t64(W["Wo"])).numpy(), rtol=0, atol=_tol(theta, T))


def _check_reduction(X, m, W, n_q, n_kv, hd, theta):
    T = X.shape[0]
    r = n_q // n_kv
    Y, O = _run(X, m, W, n_q, n_kv, hd, theta, return_o=True)
    q, k, v = qkv_lib(X, W["Wq"], W["Wk"], W["Wv"], n_q, n_kv, hd, theta, np.arange(T))
    for g in range(n_kv):
        idx = np.flatnonzero(m[:, g])
        heads = slice(g * r, (g + 1) * r)
        dropped = np.setdiff1d(np.arange(T), idx)
        assert np.all(O[dropped, heads] == 0.0)
        if idx.size:
            ref = sdpa(q[idx, heads], k[idx, g:g + 1], v[idx, g:g + 1], causal=True)
            np.testing.assert_allclose(O[idx, heads], ref, rtol=0, atol=_tol(theta, T))
            # a group's first kept token attends only to itself: its output is its v
            np.testing.assert_allclose(O[idx[0], heads], np.repeat(v[idx[0], g][None], r, 0),
                                       rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Y, O.reshape(T, -1) @ W["Wo"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("theta", [0.0, 500000.0])
@pytest.mark.parametrize("p", [0.25, 0.5, 0.8])
def test_group_reduces_to_causal_attention_over_kept_tokens(theta, p):
    T, d, n_q, n_kv, hd = 40, 32, 8, 4, 8
    W = _w(d, n_q, n_kv, hd, 4)
    rr = np.random.default_rng(int(p * 100))
    X = rr.standard_normal((T, d))
    m = (rr.random((T, n_kv)) < p).astype(np.uint8)
    _check_reduction(X, m, W, n_q, n_kv, hd, theta)


def test_brute_force_all_masks_tiny():
    T, d, n_q, n_kv, hd = 4, 6, 4, 2, 4
    W = _w(d, n_q, n_kv, hd, 5)
    X = np.random.default_rng(6).standard_normal((T, d))
    for bits in itertools.product((0, 1), repeat=T * n_kv):
        m = np.array(bits, np.uint8).reshape(T, n_kv)
        _check_reduction(X, m, W, n_q, n_kv, hd, 10000.0)


def test_all_zero_and_head_map():
    T, d, n_q, n_kv, hd = 12, 16, 8, 4, 4
    W = _w(d, n_q, n_kv, hd, 7)
    X = np.random.default_rng(8).standard_normal((T, d))
    assert np.all(_run(X, np.zeros((T, n_kv), np.uint8), W, n_q, n_kv, hd, 0.0) == 0.0)
    m = np.zeros((T, n_kv), np.uint8)
    m[:, 1] = 1
    _, O = _run(X, m, W, n_q, n_kv, hd, 0.0, return_o=True)
    live = [h for h in range(n_q) if np.any(O[:, h] != 0)]
    assert live == [2, 3]                                 # query heads 2,3 belong to KV head 1


# ----------------------------------------------------------------- decode

@pytest.mark.parametrize("theta", [0.0, 500000.0])
def test_decode_against_sdpa(theta):
    B, d, n_q, n_kv, hd, L = 5, 32, 8, 2, 8, 9
    W = _w(d, n_q, n_kv, hd, 9)
    r = n_q // n_kv
    rr = np.random.default_rng(10)
    X = rr.standard_normal((B, d))
    Kc = rr.standard_normal((B, n_kv, L + 3, hd))
    Vc = rr.standard_normal((B, n_kv, L + 3, hd))
    m = (rr.random((B, n_kv)) < 0.5).astype(np.uint8)
    m[0] = 1
    Y, Kn, Vn, O = _run(X, m, W, n_q, n_kv, hd, theta, decode=True, K_cache=Kc, V_cache=Vc,
                        kv_len=L, return_o=True)
    q, k, v = qkv_lib(X, W["Wq"], W["Wk"], W["Wv"], n_q, n_kv, hd, theta, np.full(B, L))
    for b in range(B):
        for g in range(n_kv):
            heads = slice(g * r, (g + 1) * r)
            if not m[b, g]:
                assert np.all(O[b, heads] == 0.0) and np.all(Kn[b, g] == 0.0)
                continue
            np.testing.assert_allclose(Kn[b, g], k[b, g], rtol=0, atol=_tol(theta, L + 1))
            np.testing.assert_allclose(Vn[b, g], v[b, g], rtol=1e-12, atol=1e-12)
            keys = np.concatenate([Kc[b, g, :L], k[b, g][None]])[:, None]
            vals = np.concatenate([Vc[b, g, :L], v[b, g][None]])[:, None]
            ref = sdpa(q[b:b + 1, heads], keys, vals, causal=False)[0]
            np.testing.assert_allclose(O[b, heads], ref, rtol=0, atol=_tol(theta, L + 1))
    np.testing.assert_allclose(Y, O.reshape(B, -1) @ W["Wo"], rtol=1e-12, atol=1e-12)


def test_decode_equals_last_prefill_row():
    """All-ones: decoding token L against the prefill K/V of tokens 0..L-1 equals
    row L of the prefill over L+1 tokens."""
    L, d, n_q, n_kv, hd, theta = 13, 24, 4, 2, 8, 500000.0
    W = _w(d, n_q, n_kv, hd, 11)
    X = np.random.default_rng(12).standard_normal((L + 1, d))
    Yp = _run(X, np.ones((L + 1, n_kv), np.uint8), W, n_q, n_kv, hd, theta)
    _, k, v = qkv_lib(X, W["Wq"], W["Wk"], W["Wv"], n_q, n_kv, hd, theta, np.arange(L + 1))
    Kc = np.zeros((1, n_kv, L + 1, hd))
    Vc = np.zeros((1, n_kv, L + 1, hd))
    Kc[0, :, :L] = k[:L].transpose(1, 0, 2)
    Vc[0, :, :L] = v[:L].transpose(1, 0, 2)
    Yd = _run(X[L:], np.ones((1, n_kv), np.uint8), W, n_q, n_kv, hd, theta, decode=True,
              K_cache=Kc, V_cache=Vc, kv_len=L)[0]
    np.testing.assert_allclose(Yd[0], Yp[L], rtol=0, atol=_tol(theta, L + 1))


@pytest.mark.parametrize("theta", [0.0, 500000.0])
def test_rows_option_selects_rows(theta):
    """Sampled query rows equal the same rows of the full computation."""
    T, d, n_q, n_kv, hd = 37, 24, 8, 2, 8
    W = _w(d, n_q, n_kv, hd, 13)
    rr = np.random.default_rng(14)
    X = rr.standard_normal((T, d))
    m = (rr.random((T, n_kv)) < 0.5).astype(np.uint8)
    rows = np.array([0, 3, 17, 36])
    full = _run(X, m, W, n_q, n_kv, hd, theta)
    part = _run(X, m, W, n_q, n_kv, hd, theta, rows=rows)
    np.testing.assert_allclose(part, full[rows], rtol=1e-12, atol=1e-12)


def _decode_steps_with_masked_caches(X, M, W, n_q, n_kv, hd, theta):
    """Run the sequences X [B, S, d] one token at a time from empty caches in which
    tokens that skip a group leave no entry (per-pair lengths)."""
    B, S, d = X.shape
    Kc = np.zeros((B, n_kv, S, hd))
    Vc = np.zeros((B, n_kv, S, hd))
    L = np.zeros((B, n_kv), np.int64)
    Ys = []
    for s in range(S):
        Y, Kn, Vn = attn_masked(X[:, s], M[:, s], W["Wq"], W["Wk"], W["Wv"], W["Wo"], n_q=n_q,
                                n_kv=n_kv, head_dim=hd, rope_theta=theta, decode=True,
                                K_cache=Kc, V_cache=Vc, kv_len=L, pos=s)
        for b in range(B):
            for g in range(n_kv):
                if M[b, s, g]:
                    Kc[b, g, L[b, g]] = Kn[b, g]
                    Vc[b, g, L[b, g]] = Vn[b, g]
                    L[b, g] += 1
        Ys.append(Y)
    return np.stack(Ys, axis=1), L


@pytest.mark.parametrize("theta", [0.0, 10000.0])
def test_masked_cache_decode_steps_reproduce_prefill(theta):
    """Reading R4 across decode steps: decoding a sequence token by token over caches
    that hold only the tokens which kept each group gives the prefill rows."""
    rng = np.random.default_rng(11)
    B, S, d, n_q, n_kv, hd = 3, 9, 16, 4, 2, 4
    X = rng.standard_normal((B, S, d))
    M = (rng.random((B, S, n_kv)) < 0.6).astype(np.uint8)
    W = {k: rng.standard_normal(sh) * 0.3 for k, sh in
         (("Wq", (n_q * hd, d)), ("Wk", (n_kv * hd, d)), ("Wv", (n_kv * hd, d)), ("Wo", (n_q * hd, d)))}
    Yd, L = _decode_steps_with_masked_caches(X, M, W, n_q, n_kv, hd, theta)
    np.testing.assert_array_equal(L, M.sum(axis=1))
    for b in range(B):
        Yp = attn_masked(X[b], M[b], W["Wq"], W["Wk"], W["Wv"], W["Wo"], n_q=n_q, n_kv=n_kv,
                         head_dim=hd, rope_theta=theta)
        np.testing.assert_allclose(Yd[b], Yp, rtol=1e-10, atol=1e-12)


def test_per_pair_lengths_equal_the_uniform_length():
    rng = np.random.default_rng(5)
    B, d, n_q, n_kv, hd, L0, cap = 4, 8, 4, 2, 4, 5, 7
    X = rng.standard_normal((B, d))
    M = (rng.random((B, n_kv)) < 0.7).astype(np.uint8)
    W = [rng.standard_normal(sh) for sh in ((n_q * hd, d), (n_kv * hd, d), (n_kv * hd, d), (n_q * hd, d))]
    Kc, Vc = rng.standard_normal((2, B, n_kv, cap, hd))
    a = attn_masked(X, M, *W, n_q=n_q, n_kv=n_kv, head_dim=hd, rope_theta=100.0, decode=True,
                    K_cache=Kc, V_cache=Vc, kv_len=L0)
    b = attn_masked(X, M, *W, n_q=n_q, n_kv=n_kv, head_dim=hd, rope_theta=100.0, decode=True,
                    K_cache=Kc, V_cache=Vc, kv_len=np.full((B, n_kv), L0), pos=L0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    # an out-of-range length is a dropped pair: zero output, nothing appended
    Lbad = np.full((B, n_kv), L0)
    Lbad[0, :] = cap
    c = attn_masked(X, M, *W, n_q=n_q, n_kv=n_kv, head_dim=hd, rope_theta=100.0, decode=True,
                    K_cache=Kc, V_cache=Vc, kv_len=Lbad, pos=L0)
    M0 = M.copy()
    M0[0, :] = 0
    e = attn_masked(X, M0, *W, n_q=n_q, n_kv=n_kv, head_dim=hd, rope_theta=100.0, decode=True,
                    K_cache=Kc, V_cache=Vc, kv_len=L0)
    np.testing.assert_allclose(c[0], e[0], rtol=1e-12, atol=1e-12)
    assert np.all(c[1][0] == 0) and np.all(c[2][0] == 0)


# --------------------------------------------------------- paged caches (R10)

def _scatter_pages(C, table, n_pages, fill):
    """Pool [n_pages, ps, hd] holding the contiguous caches C [B, n_kv, cap, hd] at
    the pages the table names; unnamed pages hold `fill`."""
    B, n_kv, max_pages = table.shape
    ps = C.shape[2] // max_pages
    pool = np.full((n_pages, ps, C.shape[3]), fill)
    for b, g, p in itertools.product(range(B), range(n_kv), range(max_pages)):
        if 0 <= table[b, g, p] < n_pages:
            pool[table[b, g, p]] = C[b, g, p * ps:(p + 1) * ps]
    return pool


def test_paged_gather_inverts_a_scatter():
    """Any one-to-one table: gathering the pool that the table scattered gives back
    the contiguous caches bit for bit, whatever the unused pages hold."""
    from oracle import paged_to_contiguous
    rng = np.random.default_rng(21)
    B, n_kv, max_pages, ps, hd, n_pages = 3, 2, 4, 4, 3, 30
    K, V = rng.standard_normal((2, B, n_kv, max_pages * ps, hd))
    table = rng.permutation(n_pages)[:B * n_kv * max_pages].reshape(B, n_kv, max_pages)
    L = rng.integers(0, max_pages * ps, (B, n_kv))
    Kg, Vg, Lg = paged_to_contiguous(_scatter_pages(K, table, n_pages, 7.0),
                                     _scatter_pages(V, table, n_pages, -7.0), table, L)
    np.testing.assert_array_equal(Kg, K)
    np.testing.assert_array_equal(Vg, V)
    np.testing.assert_array_equal(Lg, L)


def test_paged_gather_unmapped_and_shared_pages():
    """Unmapped entries (negative or past the pool) give zero slots, and a pair whose
    new slot is on one gets length -1; a pair whose unmapped page lies before its new
    slot keeps its length; two pairs on one page read the same rows."""
    from oracle import paged_to_contiguous
    ps, hd, n_pages = 2, 1, 3
    pool = np.arange(n_pages * ps, dtype=float).reshape(n_pages, ps, hd) + 1.0
    table = np.array([[[0, -1, 2]], [[3, 1, 1]]])           # B = 2, n_kv = 1, 3 pages
    L = np.array([[3], [4]])                               # slot 3 on page -1; slot 4 on 1
    Kg, Vg, Lg = paged_to_contiguous(pool, -pool, table, L)
    np.testing.assert_array_equal(Kg[0, 0, :, 0], [1, 2, 0, 0, 5, 6])
    np.testing.assert_array_equal(Kg[1, 0, :, 0], [0, 0, 3, 4, 3, 4])
    np.testing.assert_array_equal(Vg, -Kg)
    np.testing.assert_array_equal(Lg, [[-1], [4]])
    # a length past the capacity stays out of range
    _, _, Lg2 = paged_to_contiguous(pool, pool, table, np.array([[6], [-1]]))
    np.testing.assert_array_equal(Lg2, [[6], [-1]])


def test_paged_decode_steps_reproduce_prefill():
    """Reading R10 with R4 across steps: token-by-token decode through a pool of
    shuffled pages (each step gathers the caches, decodes, and writes the new k/v
    into the new slot's page row) gives the prefill rows."""
    from oracle import paged_to_contiguous
    rng = np.random.default_rng(13)
    B, S, d, n_q, n_kv, hd, ps = 2, 10, 16, 4, 2, 4, 4
    max_pages = S // ps + 1
    n_pages = B * n_kv * max_pages + 3
    table = rng.permutation(n_pages)[:B * n_kv * max_pages].reshape(B, n_kv, max_pages)
    X = rng.standard_normal((B, S, d))
    M = (rng.random((B, S, n_kv)) < 0.6).astype(np.uint8)
    W = _w(d, n_q, n_kv, hd, 4)
    Kp = rng.standard_normal((n_pages, ps, hd))   # stale contents past the lengths
    Vp = rng.standard_normal((n_pages, ps, hd))
    L = np.zeros((B, n_kv), np.int64)
    Ys = []
    for s in range(S):
        Kc, Vc, Le = paged_to_contiguous(Kp, Vp, table, L)
        Y, Kn, Vn = attn_masked(X[:, s], M[:, s], W["Wq"], W["Wk"], W["Wv"], W["Wo"], n_q=n_q,
                                n_kv=n_kv, head_dim=hd, rope_theta=10000.0, decode=True,
                                K_cache=Kc, V_cache=Vc, kv_len=Le, pos=s)
        Ys.append(Y)
        for b, g in zip(*np.nonzero(M[:, s])):
            Kp[table[b, g, L[b, g] // ps], L[b, g] % ps] = Kn[b, g]
            Vp[table[b, g, L[b, g] // ps], L[b, g] % ps] = Vn[b, g]
            L[b, g] += 1
    for b in range(B):
        ref = _run(X[b], M[b], W, n_q, n_kv, hd, 10000.0)
        np.testing.assert_allclose(np.stack(Ys, axis=1)[b], ref, rtol=1e-10, atol=1e-12)
