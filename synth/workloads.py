"""The synthetic workloads: shapes, distributions and mask recipes.

Every function returns a dict of numpy arrays. Float tensors are float32 holding
bf16-exact values (see ``synth.bf16_round``), masks are uint8 [T, n_groups].
Weight matrices are returned in their mathematical orientation:

* ``W_gate, W_up`` : [d_ff, d_model]   (row c produces channel c; group g = rows gG..gG+G-1)
* ``W_down``       : [d_ff, d_model]   (Y = H @ W_down; group g = rows gG..gG+G-1)
* ``Wq``           : [n_q*hd, d_model]  ``Wk, Wv`` : [n_kv*hd, d_model]
* ``Wo``           : [n_q*hd, d_model]  (Y = O @ Wo; group g = rows g*r*hd..(g+1)*r*hd-1)

The sizes named by the workloads are the Llama-3.2-3B FFN (d=3072, d_ff=8192),
and the Llama-3.1-8B FFN and attention (d=4096, d_ff=14336, 32 query heads,
8 KV heads, head_dim 128). Weights are random-init N(0, 0.02), not trained ones;
masks come from seeded router logits, Bernoulli draws or clustered prototypes in
place of learned routers.
"""
from __future__ import annotations

import numpy as np

from . import (bernoulli_mask, clustered_mask, normal, router_logits, rng,
               topk_mask)

W_STD = 0.02


def make_mask(cfg: str, T: int, n: int, keep: float, kind: str, x=None, *, tag: str = "mask",
              router_std: float | None = None) -> np.ndarray:
    """kind: 'topk' (N(0,1) logits), 'router' (top-k of x @ R), 'bernoulli',
    'clustered', 'ones', 'zeros'."""
    k = int(round(keep * n))
    if kind == "ones":
        return np.ones((T, n), np.uint8)
    if kind == "zeros":
        return np.zeros((T, n), np.uint8)
    if kind == "topk":
        logits = rng(cfg, tag + ".logits").standard_normal((T, n), dtype=np.float32)
        return topk_mask(logits, k)
    if kind == "router":
        if x is None:
            raise ValueError("router masks need x")
        std = router_std if router_std is not None else 1.0 / x.shape[1]
        return topk_mask(router_logits(x, cfg, tag + ".R", n, std), k)
    if kind == "bernoulli":
        return bernoulli_mask(cfg, tag + ".u", T, n, keep)
    if kind == "clustered":
        return clustered_mask(cfg, tag + ".proto", T, n, keep)
    raise ValueError(f"unknown mask kind {kind!r}")


def ffn_case(cfg: str, T: int, d: int, F: int, n: int, keep: float = 0.5,
             mask_kind: str = "topk", x_std: float = 1.0) -> dict:
    X = normal(cfg, "X", (T, d), x_std)
    out = dict(
        X=X,
        W_gate=normal(cfg, "W_gate", (F, d), W_STD),
        W_up=normal(cfg, "W_up", (F, d), W_STD),
        W_down=normal(cfg, "W_down", (F, d), W_STD),
        mask=make_mask(cfg, T, n, keep, mask_kind, X, tag="ffn_mask"),
    )
    out["meta"] = dict(T=T, d=d, F=F, n=n, keep=keep, mask_kind=mask_kind)
    return out


def attn_weights(cfg: str, d: int, n_q: int, n_kv: int, hd: int) -> dict:
    return dict(
        Wq=normal(cfg, "Wq", (n_q * hd, d), W_STD),
        Wk=normal(cfg, "Wk", (n_kv * hd, d), W_STD),
        Wv=normal(cfg, "Wv", (n_kv * hd, d), W_STD),
        Wo=normal(cfg, "Wo", (n_q * hd, d), W_STD),
    )


def attn_case(cfg: str, T: int, d: int = 4096, n_q: int = 32, n_kv: int = 8, hd: int = 128,
              keep: float = 0.5, mask_kind: str = "topk", *, decode: bool = False,
              kv_len: int = 0, kv_cap: int = 0) -> dict:
    """Prefill: T tokens at positions 0..T-1.  Decode: T = batch, one new token per
    sequence at position kv_len, caches [T, n_kv, kv_cap, hd] ~ N(0,1) whose first
    kv_len slots are valid."""
    X = normal(cfg, "X", (T, d))
    out = dict(X=X, mask=make_mask(cfg, T, n_kv, keep, mask_kind, X, tag="attn_mask"))
    out.update(attn_weights(cfg, d, n_q, n_kv, hd))
    if decode:
        if not 0 <= kv_len < kv_cap:
            raise ValueError("decode needs 0 <= kv_len < kv_cap")
        out["K_cache"] = normal(cfg, "K_cache", (T, n_kv, kv_cap, hd))
        out["V_cache"] = normal(cfg, "V_cache", (T, n_kv, kv_cap, hd))
    out["meta"] = dict(T=T, d=d, n_q=n_q, n_kv=n_kv, hd=hd, keep=keep, mask_kind=mask_kind,
                       decode=decode, kv_len=kv_len, kv_cap=kv_cap)
    return out


def paged_cache(cfg: str, B: int, n_kv: int, page_size: int, max_pages: int, hd: int = 128, *,
                spare_pages: int = 5, unmapped: float = 0.0, shared_pages: int = 0) -> dict:
    """A paged K/V cache for B sequences x n_kv groups: pools [n_pages, page_size, hd]
    ~ N(0,1), a page table [B, n_kv, max_pages] int32 that deals the pages out in a
    seeded random order (spare_pages pages stay unused), and per-pair lengths
    kv_len [B, n_kv] int32 uniform over the capacity (the first pair at 0 and the last
    at capacity - 1 when nothing is shared).

    unmapped: the fraction of table entries replaced by unmapped ones (half -1, half
    past the pool).  shared_pages: every pair's first shared_pages entries name the
    first pair's, and every length is at least shared_pages * page_size, so the new
    slots fall past the shared pages."""
    r = rng(cfg, "page_table")
    n_pages = B * n_kv * max_pages + spare_pages
    table = r.permutation(n_pages)[:B * n_kv * max_pages].reshape(B, n_kv, max_pages)
    if shared_pages:
        table[:, :, :shared_pages] = table[0, 0, :shared_pages]
    if unmapped:
        hit = r.random(table.shape) < unmapped
        table[hit] = np.where(r.random(table.shape) < 0.5, -1, n_pages + 3)[hit]
    cap = max_pages * page_size
    lo = shared_pages * page_size
    L = rng(cfg, "kv_len").integers(lo, cap, size=(B, n_kv))
    if not shared_pages:
        L.flat[0], L.flat[-1] = 0, cap - 1
    return dict(K_pool=normal(cfg, "K_pool", (n_pages, page_size, hd)),
                V_pool=normal(cfg, "V_pool", (n_pages, page_size, hd)),
                page_table=table.astype(np.int32), kv_len=L.astype(np.int32),
                meta=dict(B=B, n_kv=n_kv, page_size=page_size, max_pages=max_pages,
                          n_pages=n_pages, unmapped=unmapped, shared_pages=shared_pages))


def layer_case(cfg: str, T: int, d: int = 4096, F: int = 14336, n_ffn: int = 112,
               n_q: int = 32, n_kv: int = 8, hd: int = 128, keep: float = 0.5,
               mask_kind: str = "router", *, decode: bool = False, kv_len: int = 0,
               kv_cap: int = 0, rope_theta: float = 500000.0, eps: float = 1e-5,
               attn_keep: float | None = None) -> dict:
    """A Llama-style decoder layer: RMSNorm weights are 1, masks come from the layer
    input x (router kind: R std 1/64), K/V caches ~ N(0,1) in decode."""
    X = normal(cfg, "X", (T, d))
    rstd = 1.0 / 64.0
    out = dict(
        X=X,
        attn_mask=make_mask(cfg, T, n_kv, keep if attn_keep is None else attn_keep, mask_kind, X,
                            tag="attn_mask", router_std=rstd),
        ffn_mask=make_mask(cfg, T, n_ffn, keep, mask_kind, X, tag="ffn_mask", router_std=rstd),
        rms1=np.ones(d, np.float32),
        rms2=np.ones(d, np.float32),
        W_gate=normal(cfg, "W_gate", (F, d), W_STD),
        W_up=normal(cfg, "W_up", (F, d), W_STD),
        W_down=normal(cfg, "W_down", (F, d), W_STD),
    )
    out.update(attn_weights(cfg, d, n_q, n_kv, hd))
    if decode:
        if not 0 <= kv_len < kv_cap:
            raise ValueError("decode needs 0 <= kv_len < kv_cap")
        out["K_cache"] = normal(cfg, "K_cache", (T, n_kv, kv_cap, hd))
        out["V_cache"] = normal(cfg, "V_cache", (T, n_kv, kv_cap, hd))
    out["meta"] = dict(T=T, d=d, F=F, n_ffn=n_ffn, n_q=n_q, n_kv=n_kv, hd=hd, keep=keep,
                       mask_kind=mask_kind, decode=decode, kv_len=kv_len, kv_cap=kv_cap,
                       rope_theta=rope_theta, eps=eps)
    return out


# ------------------------------------------------------------ named workloads

def tiny_ffn():
    """SwiGLU FFN d=256, d_ff=1024 in 16 groups of 64, T=64, keep 8 of 16."""
    return ffn_case("tiny_ffn", 64, 256, 1024, 16, 0.5, "topk")


def ffn_prefill_3b(T: int = 4096, ffn_group: int = 128):
    """Llama-3.2-3B FFN prefill: d=3072, d_ff=8192 in groups of ``ffn_group`` channels
    (64 groups of 128 by default), keeping half of them by top-k of x @ R,
    R [3072, n] ~ N(0, 1/3072).  Inputs and weights do not depend on the group size."""
    if 8192 % ffn_group:
        raise ValueError("ffn_group must divide 8192")
    return ffn_case("ffn_prefill_3b", T, 3072, 8192, 8192 // ffn_group, 0.5, "router")


def ffn_decode_8b(B: int):
    """Llama-3.1-8B FFN decode: d=4096, d_ff=14336 in 112 groups of 128, keep 56."""
    return ffn_case(f"ffn_decode_8b_B{B}", B, 4096, 14336, 112, 0.5, "topk")


def attn_prefill_8b(T: int = 2048):
    return attn_case("attn_prefill_8b", T, keep=0.5, mask_kind="topk")


def attn_decode_8b(B: int = 16, L: int = 4096):
    return attn_case("attn_decode_8b", B, keep=0.5, mask_kind="topk", decode=True,
                     kv_len=L, kv_cap=L + 1)


def layer_8b(T: int, *, decode: bool = False, L: int = 0, keep: float = 0.5, kind: str = "router",
             ffn_group: int = 128, attn_keep: float | None = None):
    """The 8B layer; ``ffn_group`` channels per FFN group (d_ff = 14336 in 14336 / ffn_group
    groups).  Inputs and weights do not depend on the group size, only the FFN mask does.
    ``attn_keep`` gives the attention mask its own keep ratio (``keep`` is then the FFN's)."""
    if 14336 % ffn_group:
        raise ValueError("ffn_group must divide 14336")
    name = f"layer_8b_{'dec' if decode else 'pre'}_{kind}_{int(round(keep * 100))}"
    return layer_case(name, T, n_ffn=14336 // ffn_group, keep=keep, mask_kind=kind, decode=decode,
                      kv_len=L, kv_cap=(L + 1) if decode else 0, attn_keep=attn_keep)
