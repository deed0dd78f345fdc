"""Dense CPU oracle of WIDE's masked dynamic-width execution (test infrastructure).

TEST INFRASTRUCTURE ONLY: see ``oracle/__init__.py`` for who may use it.

Sources (the pages about "WIDE: Boosting Adaptive LLM Inference via Token-level
Dynamic Width Pruning"):

* [abstract]     the English abstract (arxivdaily.com, insight.artgrammer.co.kr and
                 franklineh.com pages): each token picks attention-head groups and
                 FFN-channel groups; the co-design splits acceleration into mask
                 reordering, block-level skipping and intra-block skipping.
* [gist §2A]     gist.science technical summary (zh and ja), section 2.A
                 "fine-grained token-level routing": attention units are head
                 groups aligned with GQA; FFN units are contiguous channel groups of
                 the intermediate dimension D'; a router gives one binary
                 execute/skip decision per group.
* [gist §2B]     same page, section 2.B "unified mask-reordering preprocessing": per
                 routing group the binary mask is sorted along the token dimension M
                 so active tokens form a contiguous prefix, with no explicit
                 gather-scatter and no token-specific sparse tensors.
* [gist §2C]     same page, section 2.C "pruning-kernel co-design": a tile whose
                 token block is inactive for a group exits (l=0); inactive load
                 packets (l=1) and MMA fragments (l=2) are skipped.  Skipping only
                 removes work whose result is unused, so the masked layer equals
                 the dense layer with dropped groups zeroed.

Readings taken where the pages are silent (each one is listed again in the
design notes):

* R1 reorder tie rule: the sort is stable, ascending token index inside the
  active and inactive classes.  Bits pack little-endian (group 64w+j -> bit j of
  word w); nonzero mask bytes mean "keep"; tile unions are ascending, padded -1.
* R2 FFN activation: Llama SwiGLU, H = silu(X W_gate^T) * (X W_up^T), no bias.
* R3 GQA index map: query head h belongs to KV group h // r, r = n_q / n_kv.
* R4 attention over kept groups: a query kept in group g attends to the earlier
  (and its own) tokens that also kept g; tokens that skipped g have no K/V in g.
  Scale 1/sqrt(head_dim).  Outputs of skipped groups are exactly zero.
* R5 decode: the K/V cache of each (sequence, group) holds kv_len valid entries;
  a new token kept in g attends to all of them plus itself and is appended at slot
  kv_len; a skipped (sequence, group) writes nothing and outputs zero.  Across
  decode steps R4 means the caches hold only the tokens that kept the group, so
  each (sequence, group) has its own length (kv_len [B, n_kv]); the new token's
  RoPE position is then a separate argument.  A length outside [0, kv_cap) makes
  the pair write nothing and output zero.
* R6 layer: pre-norm Llama block, RMSNorm x / sqrt(mean(x^2) + eps) * gamma,
  rotate-half RoPE with angle pos * theta^(-2i/hd), no frequency scaling.
* R9 router: a linear router without bias, logits = X R^T with R group-major
  [n, d]; a token keeps the k groups with the largest logits, ties to the lower
  group index (-0.0 and +0.0 are equal).  The pages say only that a router gives
  one binary execute/skip decision per group [gist §2A] and that routing is
  learned per token [abstract]; the router's form and the top-k rule are the
  plainest reading of a fixed keep ratio.
* R10 paged masked cache: the pages name a paged layout for the decode caches
  but give no page format.  The one taken here: K and V pools [n_pages, page_size,
  hd]; a page table [B, n_kv, max_pages] gives the page of each page_size-slot
  stretch of a (sequence, group) cache.  A slot on an unmapped page (entry outside
  [0, n_pages)) holds zeros; a pair whose new slot is on one is treated like an
  out-of-range length (R5).  Everything else is R5 on the gathered caches.
"""
from __future__ import annotations

import numpy as np


def _f(a, dtype):
    return np.asarray(a, dtype=dtype)


# ------------------------------------------------------------------ reorder

def mask_reorder(mask, tile_m: int) -> dict:
    """Mask reordering [gist §2B], with reading R1.

    For every group g the tokens are sorted on the binary key (0 = kept first),
    stably, which puts the active tokens in a contiguous prefix of length
    ``group_count[g]``.  ``group_rank`` is the inverse permutation.  For every tile
    of ``tile_m`` consecutive tokens, ``tile_groups`` lists (ascending) the groups
    that at least one token of the tile keeps; a (tile, group) block outside that
    list is the block that [gist §2C] l=0 skips.
    """
    m = np.asarray(mask) != 0
    if m.ndim != 2:
        raise ValueError("mask must be [T, n_groups]")
    if tile_m < 1:
        raise ValueError("tile_m must be >= 1")
    T, n = m.shape
    nw = (n + 63) // 64

    packed = np.zeros((T, nw), np.uint64)
    for g in range(n):
        w, j = divmod(g, 64)
        packed[:, w] |= m[:, g].astype(np.uint64) << np.uint64(j)

    count = np.zeros(n, np.int32)
    perm = np.zeros((n, T), np.int32)
    rank = np.zeros((n, T), np.int32)
    for g in range(n):
        active = [t for t in range(T) if m[t, g]]
        inactive = [t for t in range(T) if not m[t, g]]
        count[g] = len(active)
        order = active + inactive
        perm[g] = order
        for i, t in enumerate(order):
            rank[g, t] = i

    n_tiles = (T + tile_m - 1) // tile_m
    tile_count = np.zeros(n_tiles, np.int32)
    tile_groups = np.full((n_tiles, n), -1, np.int32)
    for i in range(n_tiles):
        rows = m[i * tile_m:min(T, (i + 1) * tile_m)]
        kept = [g for g in range(n) if rows[:, g].any()]
        tile_count[i] = len(kept)
        tile_groups[i, :len(kept)] = kept

    return dict(packed=packed, group_count=count, group_perm=perm, group_rank=rank,
                tile_count=tile_count, tile_groups=tile_groups)


# ---------------------------------------------------------------------- FFN

def _silu(a):
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def ffn_masked(X, mask, W_gate, W_up, W_down, *, dtype=np.float64, return_h: bool = False):
    """Masked SwiGLU FFN: FFN-channel groups of D' [gist §2A], reading R2.

    X [T, d]; mask [T, n]; W_gate, W_up, W_down [F, d] with group g owning
    channels gG .. gG+G-1 (G = F / n).  Dense gate/up, SwiGLU, zero the channels
    of every group the token drops, then the down projection Y = H @ W_down.
    """
    X, Wg, Wu, Wd = (_f(a, dtype) for a in (X, W_gate, W_up, W_down))
    m = np.asarray(mask) != 0
    T, d = X.shape
    F = Wg.shape[0]
    n = m.shape[1]
    if F % n:
        raise ValueError("d_ff must be a multiple of n_groups")
    G = F // n
    A = X @ Wg.T
    B = X @ Wu.T
    H = _silu(A) * B
    H = np.where(np.repeat(m, G, axis=1), H, 0.0)
    Y = H @ Wd
    return (Y, H) if return_h else Y


# ---------------------------------------------------------------- attention

def rmsnorm(x, gamma, eps: float, *, dtype=np.float64):
    """RMSNorm of the Llama block (reading R6)."""
    x = _f(x, dtype)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _f(gamma, dtype)


def rope(x, pos, theta: float, *, dtype=np.float64):
    """Rotate-half RoPE (reading R6).  x [..., T, heads, hd], pos [T]."""
    x = _f(x, dtype)
    hd = x.shape[-1]
    half = hd // 2
    inv = float(theta) ** (-(2.0 * np.arange(half, dtype=dtype)) / hd)
    ang = np.asarray(pos, dtype)[:, None] * inv[None, :]          # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _softmax_rows(S):
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    return P / P.sum(axis=-1, keepdims=True)


def attn_masked(X, mask, Wq, Wk, Wv, Wo, *, n_q: int, n_kv: int, head_dim: int,
                rope_theta: float = 0.0, decode: bool = False, K_cache=None, V_cache=None,
                kv_len=0, pos=None, dtype=np.float64, return_o: bool = False, rows=None):
    """Masked attention sublayer: GQA-aligned head groups [gist §2A], readings R3-R5.

    One group = one KV head and its r = n_q / n_kv query heads.  Projections are
    computed densely and the columns of dropped groups zeroed; the attention core
    follows R4 (prefill, positions 0..T-1, causal) or R5 (decode, one new token per
    sequence at position kv_len); Y = O @ Wo with O zero in dropped groups.

    Prefill returns Y [T, d]; with ``rows`` (prefill only) just those query rows are
    produced, Y [len(rows), d], from the same keys and values.  Decode returns
    (Y, K_new, V_new) where K_new, V_new
    [B, n_kv, hd] are the (roped) keys/values appended at slot kv_len for the kept
    (sequence, group) pairs (zero rows elsewhere; nothing is appended there).
    ``kv_len`` is one length for the batch or an array [B, n_kv] of per-pair
    lengths (then ``pos``, the new tokens' position, is required).
    """
    X, Wq, Wk, Wv, Wo = (_f(a, dtype) for a in (X, Wq, Wk, Wv, Wo))
    keep = np.asarray(mask) != 0                                  # [T, n_kv]
    T = X.shape[0]
    hd = head_dim
    if n_q % n_kv:
        raise ValueError("n_q must be a multiple of n_kv")
    r = n_q // n_kv
    Eq = np.repeat(keep, r * hd, axis=1)
    Ek = np.repeat(keep, hd, axis=1)
    if rows is not None and not decode:
        Q = np.zeros((T, n_q, hd), dtype)
        R_ = np.asarray(rows)
        Q[R_] = np.where(Eq[R_], X[R_] @ Wq.T, 0.0).reshape(len(R_), n_q, hd)
    else:
        Q = np.where(Eq, X @ Wq.T, 0.0).reshape(T, n_q, hd)
    K = np.where(Ek, X @ Wk.T, 0.0).reshape(T, n_kv, hd)
    V = np.where(Ek, X @ Wv.T, 0.0).reshape(T, n_kv, hd)
    L = np.asarray(kv_len)
    if decode and L.ndim == 2 and pos is None:
        raise ValueError("per-pair kv_len needs pos")
    pos = np.full(T, int(L) if pos is None else pos) if decode else np.arange(T)
    if rope_theta:
        if rows is not None and not decode:
            R_ = np.asarray(rows)
            Q[R_] = rope(Q[R_], pos[R_], rope_theta, dtype=dtype)
        else:
            Q = rope(Q, pos, rope_theta, dtype=dtype)
        K = rope(K, pos, rope_theta, dtype=dtype)
    scale = 1.0 / np.sqrt(hd)
    O = np.zeros((T, n_q, hd), dtype)

    if not decode:
        R = np.arange(T) if rows is None else np.asarray(rows)
        causal = np.arange(T)[None, :] <= R[:, None]               # key s <= query t
        OR = np.zeros((len(R), n_q, hd), dtype)
        for h in range(n_q):
            g = h // r
            sel = keep[R, g]
            if not sel.any():
                continue
            allowed = causal[sel] & keep[None, :, g]
            S = (Q[R[sel], h] @ K[:, g].T) * scale
            P = _softmax_rows(np.where(allowed, S, -np.inf))
            OR[sel, h] = P @ V[:, g]
        Y = OR.reshape(len(R), n_q * hd) @ Wo
        return (Y, OR) if return_o else Y

    Kc = _f(K_cache, dtype)
    Vc = _f(V_cache, dtype)
    cap = Kc.shape[2]
    for b in range(T):
        for g in range(n_kv):
            if not keep[b, g]:
                continue
            lb = int(L[b, g]) if L.ndim == 2 else int(L)
            if not 0 <= lb < cap:  # out-of-range length: nothing appended, zero output
                K[b, g] = 0.0
                V[b, g] = 0.0
                continue
            keys = np.concatenate([Kc[b, g, :lb], K[b, g][None]], axis=0)
            vals = np.concatenate([Vc[b, g, :lb], V[b, g][None]], axis=0)
            for h in range(g * r, (g + 1) * r):
                p = _softmax_rows(((keys @ Q[b, h]) * scale)[None])[0]
                O[b, h] = p @ vals
    Y = O.reshape(T, n_q * hd) @ Wo
    out = (Y, K, V)
    return out + (O,) if return_o else out


def paged_to_contiguous(K_pool, V_pool, page_table, kv_len):
    """Reading R10: the (sequence, group) caches a paged pool holds, gathered into
    the contiguous layout of R5, and the lengths R5 then takes.

    K_pool, V_pool [n_pages, page_size, hd]; page_table [B, n_kv, max_pages];
    kv_len [B, n_kv].  Returns (K_cache, V_cache, kv_len_eff) with caches
    [B, n_kv, max_pages * page_size, hd]: slot s of pair (b, g) is row
    s % page_size of page page_table[b, g, s // page_size], or zeros when that
    entry is outside [0, n_pages).  kv_len_eff is kv_len, except -1 (out of range)
    for a pair whose new slot kv_len[b, g] lies on an unmapped page."""
    n_pages, ps = K_pool.shape[0], K_pool.shape[1]
    table = np.asarray(page_table)
    B, n_kv, max_pages = table.shape
    cap = max_pages * ps
    K = np.zeros((B, n_kv, cap) + K_pool.shape[2:], K_pool.dtype)
    V = np.zeros_like(K)
    L = np.array(kv_len, dtype=np.int64, copy=True)
    for b in range(B):
        for g in range(n_kv):
            for p in range(max_pages):
                e = int(table[b, g, p])
                if 0 <= e < n_pages:
                    K[b, g, p * ps:(p + 1) * ps] = K_pool[e]
                    V[b, g, p * ps:(p + 1) * ps] = V_pool[e]
            lb = int(L[b, g])
            if 0 <= lb < cap and not 0 <= int(table[b, g, lb // ps]) < n_pages:
                L[b, g] = -1
    return K, V, L


# -------------------------------------------------------------------- layer

def layer_masked(X, attn_mask, ffn_mask, W: dict, *, n_q: int, n_kv: int, head_dim: int,
                 n_ffn: int, rope_theta: float, eps: float, decode: bool = False,
                 K_cache=None, V_cache=None, kv_len=0, pos=None, dtype=np.float64,
                 return_parts: bool = False, rows=None):
    """Pre-norm decoder layer with masked attention and masked FFN (reading R6).

    u = RMSNorm(x; rms1); h = x + Attn(u; attn_mask); w = RMSNorm(h; rms2);
    y = h + FFN(w; ffn_mask).  W holds rms1, rms2, Wq, Wk, Wv, Wo, W_gate, W_up,
    W_down.  ``n_ffn`` is the FFN group count (the mask's width).  With ``rows``
    (prefill only) just those token rows of y are produced.  In decode, ``kv_len``
    and ``pos`` are passed to the attention sublayer as they are (one length, or
    per-(sequence, group) lengths with the new tokens' position, reading R5).
    """
    X = _f(X, dtype)
    if np.asarray(ffn_mask).shape[1] != n_ffn:
        raise ValueError("ffn_mask width must equal n_ffn")
    u = rmsnorm(X, W["rms1"], eps, dtype=dtype)
    att = attn_masked(u, attn_mask, W["Wq"], W["Wk"], W["Wv"], W["Wo"], n_q=n_q, n_kv=n_kv,
                      head_dim=head_dim, rope_theta=rope_theta, decode=decode,
                      K_cache=K_cache, V_cache=V_cache, kv_len=kv_len, pos=pos, dtype=dtype,
                      rows=None if decode else rows)
    a = att[0] if decode else att
    R = slice(None) if (rows is None or decode) else np.asarray(rows)
    h = X[R] + a
    w = rmsnorm(h, W["rms2"], eps, dtype=dtype)
    f = ffn_masked(w, np.asarray(ffn_mask)[R], W["W_gate"], W["W_up"], W["W_down"], dtype=dtype)
    y = h + f
    parts = dict(u=u, a=a, h=h, w=w, f=f)
    if decode:
        parts.update(K_new=att[1], V_new=att[2])
    return (y, parts) if return_parts else y


# ------------------------------------------------------------------- router

def router_topk(X, R, k: int, *, logits=None, dtype=np.float64) -> dict:
    """Router and top-k selection, the step before the path (reading R9).

    logits[t, g] = sum_j X[t, j] R[g, j].  Token t keeps group g when fewer than k
    groups rank before g, where g' ranks before g if its logit is larger, or equal
    with a lower index.  With ``logits`` given, the selection is taken on those
    values instead (the decision is then made on exactly the numbers another
    implementation produced).  Returns logits, mask uint8 [T, n] and packed
    little-endian bit words [T, ceil(n/64)].
    """
    if logits is None:
        X = _f(X, dtype)
        R = _f(R, dtype)
        if X.ndim != 2 or R.ndim != 2 or X.shape[1] != R.shape[1]:
            raise ValueError("X must be [T, d] and R [n, d]")
        L = X @ R.T
    else:
        L = _f(logits, dtype)
    T, n = L.shape
    if not 0 <= k <= n:
        raise ValueError("router_topk: k out of range")
    mask = np.zeros((T, n), np.uint8)
    for t in range(T):
        row = L[t]
        for g in range(n):
            before = 0
            for h in range(n):
                if row[h] > row[g] or (row[h] == row[g] and h < g):
                    before += 1
            if before < k:
                mask[t, g] = 1
    nw = (n + 63) // 64
    packed = np.zeros((T, nw), np.uint64)
    for g in range(n):
        w, j = divmod(g, 64)
        packed[:, w] |= mask[:, g].astype(np.uint64) << np.uint64(j)
    return dict(logits=L, mask=mask, packed=packed)
