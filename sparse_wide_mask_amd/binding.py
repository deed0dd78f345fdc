"""ctypes binding of libwide (include/wide.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwide.so")

WIDE_OK, WIDE_EINVAL, WIDE_EUNSUPPORTED, WIDE_EWORKSPACE, WIDE_EHIP = range(5)
WIDE_FLAG_FFN_TOKEN_SORT = 0x2
WIDE_PREFILL, WIDE_DECODE = 0, 1

_p = C.c_void_p
_i = C.c_int
_sz = C.c_size_t


class WideAttnCfg(C.Structure):
    _fields_ = [("n_q_heads", _i), ("n_kv_heads", _i), ("head_dim", _i), ("rope_theta", C.c_float)]


class WideLayerWeights(C.Structure):
    _fields_ = [(k, _p) for k in ("rms1", "Wq", "Wk", "Wv", "Wo_packed", "rms2", "W_gate", "W_up",
                                  "W_down_packed")]


class WideLayerRouter(C.Structure):
    _fields_ = [("R_attn_packed", _p), ("R_ffn_packed", _p), ("k_attn", _i), ("k_ffn", _i)]


class WideLayerCfg(C.Structure):
    _fields_ = [("d_model", _i), ("d_ff", _i), ("n_ffn_groups", _i), ("attn", WideAttnCfg),
                ("rms_eps", C.c_float)]


_SIGS = {
    "wide_status_string": ([_i], C.c_char_p),
    "wide_version": ([], _i),
    "wide_mask_reorder": ([_p, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p], _i),
    "wide_mask_reorder_packed": ([_p, _i, _i, _i, _p, _p, _p, _p, _p, _p], _i),
    "wide_pack_kmajor": ([_p, _i, _i, _i, _p, _p], _i),
    "wide_router_topk": ([_p, _p, _i, _i, _i, _i, _p, _p, _p, _p], _i),
    "wide_pack_router": ([_p, _i, _i, _p, _p], _i),
    "wide_ffn_masked_workspace": ([_i, _i, _i, _i, _i], _sz),
    "wide_ffn_masked": ([_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _sz, C.c_uint32, _p], _i),
    "wide_ffn_masked_f32_workspace": ([_i, _i, _i, _i], _sz),
    "wide_ffn_masked_f32": ([_p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _p, _sz, C.c_uint32, _p], _i),
    "wide_ffn_masked_noalloc": ([_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, C.c_uint32, _p], _i),
    "wide_attn_proj_masked_workspace": ([_i, _i, C.POINTER(WideAttnCfg), _i, _i], _sz),
    "wide_attn_proj_masked": ([_p, _p, _p, _p, _p, _p, _i, _i, C.POINTER(WideAttnCfg), _i, _p, _p,
                               _i, _i, _p, _p, _sz, C.c_uint32, _p], _i),
    "wide_layer_masked_workspace": ([_i, C.POINTER(WideLayerCfg), _i, _i], _sz),
    "wide_attn_decode_masked_cache": ([_p, _p, _p, _p, _p, _p, _i, _i, C.POINTER(WideAttnCfg), _p,
                                       _p, _i, _p, _i, _p, _p, _sz, C.c_uint32, _p], _i),
    "wide_attn_decode_masked_paged": ([_p, _p, _p, _p, _p, _p, _i, _i, C.POINTER(WideAttnCfg),
                                       _p, _p, _i, _i, _p, _i, _p, _i, _p, _p, _sz, C.c_uint32,
                                       _p], _i),
    "wide_trace_enable": ([_i], _i),
    "wide_trace_collect": ([], _i),
    "wide_trace_get": ([_i, C.c_char_p, _i, C.POINTER(_i), C.POINTER(C.c_double)], _i),
    "wide_trace_reset": ([], None),
    "wide_layer_masked": ([_p, _p, _p, C.POINTER(WideLayerWeights), C.POINTER(WideLayerCfg), _i, _i,
                           _p, _p, _i, _i, _p, _p, _sz, C.c_uint32, _p], _i),
    "wide_layer_masked_routed": ([_p, C.POINTER(WideLayerRouter), C.POINTER(WideLayerWeights),
                                  C.POINTER(WideLayerCfg), _i, _i, _p, _p, _i, _i, _p, _p, _p, _p,
                                  _sz, C.c_uint32, _p], _i),
    "wide_layer_decode_masked_cache": ([_p, _p, _p, C.POINTER(WideLayerWeights),
                                        C.POINTER(WideLayerCfg), _i, _p, _p, _i, _p, _i, _p, _p,
                                        _sz, C.c_uint32, _p], _i),
    "wide_layer_decode_masked_paged": ([_p, _p, _p, C.POINTER(WideLayerWeights),
                                        C.POINTER(WideLayerCfg), _i, _p, _p, _i, _i, _p, _i, _p,
                                        _i, _p, _p, _sz, C.c_uint32, _p], _i),
}

_lib = None


def lib() -> C.CDLL:
    """Load libwide.so (built by ``__graft_entry__.build()``); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libwide.so not built ({LIB_PATH}); run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


class WideError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().wide_status_string(status).decode()
        super().__init__(f"{fn} failed: status {status} ({msg})")


def _check(fn: str, status: int):
    if status != WIDE_OK:
        raise WideError(fn, status)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _mode(mode) -> int:
    if mode in ("prefill", WIDE_PREFILL):
        return WIDE_PREFILL
    if mode in ("decode", WIDE_DECODE):
        return WIDE_DECODE
    raise ValueError(f"mode must be 'prefill' or 'decode', got {mode!r}")


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


# -------------------------------------------------------------------- trace

def trace_enable(on: bool = True):
    lib().wide_trace_enable(1 if on else 0)


def trace_reset():
    lib().wide_trace_reset()


def trace_collect() -> dict:
    """{kernel name: (launches, total ms)} of the launches recorded so far."""
    L = lib()
    n = L.wide_trace_collect()
    if n < 0:
        raise RuntimeError("wide_trace_collect: HIP event query failed")
    out = {}
    buf = C.create_string_buffer(256)
    for i in range(n):
        k, ms = _i(), C.c_double()
        if L.wide_trace_get(i, buf, 256, C.byref(k), C.byref(ms)) == 0:
            out[buf.value.decode()] = (k.value, ms.value)
    return out


# ------------------------------------------------------------------ reorder

def mask_reorder(mask: torch.Tensor, tile_m: int, out: dict | None = None,
                 unions: bool = True) -> dict:
    """wide_mask_reorder on a uint8 [T, n] device mask; returns the six outputs
    (four without tile unions: unions=False passes null tile_count / tile_groups)."""
    _dev(mask, torch.uint8, "mask")
    T, n = mask.shape
    dev = mask.device
    nw = (n + 63) // 64
    nt = -(-T // tile_m) if T else 0
    if out is None:
        out = dict(
            packed=torch.empty((T, nw), dtype=torch.int64, device=dev),
            group_count=torch.empty(n, dtype=torch.int32, device=dev),
            group_perm=torch.empty((n, T), dtype=torch.int32, device=dev),
            group_rank=torch.empty((n, T), dtype=torch.int32, device=dev),
        )
        if unions:
            out["tile_count"] = torch.empty(nt, dtype=torch.int32, device=dev)
            out["tile_groups"] = torch.empty((nt, n), dtype=torch.int32, device=dev)
    tc = _ptr(out["tile_count"]) if unions else None
    tg = _ptr(out["tile_groups"]) if unions else None
    st = lib().wide_mask_reorder(_ptr(mask), T, n, tile_m, _ptr(out["packed"]),
                                 _ptr(out["group_count"]), _ptr(out["group_perm"]),
                                 _ptr(out["group_rank"]), tc, tg, _stream())
    _check("wide_mask_reorder", st)
    return out


def mask_reorder_packed(packed: torch.Tensor, n_groups: int, tile_m: int,
                        out: dict | None = None) -> dict:
    """wide_mask_reorder_packed on packed mask words [T, ceil(n/64)] (int64 view of
    the uint64 words, e.g. router_topk's "packed"); returns the five reorder outputs."""
    _dev(packed, torch.int64, "packed")
    T = packed.shape[0]
    n = n_groups
    if packed.shape[1] != (n + 63) // 64:
        raise ValueError("packed must be [T, ceil(n_groups / 64)]")
    dev = packed.device
    nt = -(-T // tile_m) if T else 0
    if out is None:
        out = dict(
            group_count=torch.empty(n, dtype=torch.int32, device=dev),
            group_perm=torch.empty((n, T), dtype=torch.int32, device=dev),
            group_rank=torch.empty((n, T), dtype=torch.int32, device=dev),
            tile_count=torch.empty(nt, dtype=torch.int32, device=dev),
            tile_groups=torch.empty((nt, n), dtype=torch.int32, device=dev),
        )
    st = lib().wide_mask_reorder_packed(_ptr(packed), T, n, tile_m, _ptr(out["group_count"]),
                                        _ptr(out["group_perm"]), _ptr(out["group_rank"]),
                                        _ptr(out["tile_count"]), _ptr(out["tile_groups"]),
                                        _stream())
    _check("wide_mask_reorder_packed", st)
    return out


def pack_router(R: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """wide_pack_router: R [n, d] bf16 -> fragment order, returned as [ceil(n/16)*16, d]."""
    _dev(R, torch.bfloat16, "R")
    n, d = R.shape
    if out is None:
        out = torch.empty(((n + 15) // 16 * 16, d), dtype=torch.bfloat16, device=R.device)
    _check("wide_pack_router", lib().wide_pack_router(_ptr(R), n, d, _ptr(out), _stream()))
    return out


def router_topk(X: torch.Tensor, R_packed: torch.Tensor, k: int, n_groups: int, *,
                return_logits: bool = False, out: dict | None = None) -> dict:
    """wide_router_topk: X [T, d] bf16 and the router weights packed by pack_router ->
    mask uint8 [T, n], packed [T, nw] (int64 view of the uint64 words) and, with
    ``return_logits``, fp32 logits [T, n]."""
    _dev(X, torch.bfloat16, "X")
    _dev(R_packed, torch.bfloat16, "R_packed")
    T, d = X.shape
    n = n_groups
    if tuple(R_packed.shape) != ((n + 15) // 16 * 16, d):
        raise ValueError("R_packed must be pack_router of an [n_groups, d_model] R")
    dev = X.device
    if out is None:
        out = dict(mask=torch.empty((T, n), dtype=torch.uint8, device=dev),
                   packed=torch.empty((T, (n + 63) // 64), dtype=torch.int64, device=dev))
        if return_logits:
            out["logits"] = torch.empty((T, n), dtype=torch.float32, device=dev)
    st = lib().wide_router_topk(_ptr(X), _ptr(R_packed), T, d, n, k, _ptr(out.get("logits")),
                                _ptr(out["mask"]), _ptr(out.get("packed")), _stream())
    _check("wide_router_topk", st)
    return out


def pack_kmajor(W: torch.Tensor, n_groups: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """wide_pack_kmajor: W [n*G, d] bf16 -> [n, d, G]."""
    _dev(W, torch.bfloat16, "W")
    K, d = W.shape
    if K % n_groups:
        raise ValueError("rows of W must be a multiple of n_groups")
    G = K // n_groups
    if out is None:
        out = torch.empty((n_groups, d, G), dtype=torch.bfloat16, device=W.device)
    _check("wide_pack_kmajor", lib().wide_pack_kmajor(_ptr(W), n_groups, G, d, _ptr(out), _stream()))
    return out


# ---------------------------------------------------------------------- FFN

def ffn_masked_workspace(T, d_model, d_ff, n_groups, mode="prefill") -> int:
    return int(lib().wide_ffn_masked_workspace(T, d_model, d_ff, n_groups, _mode(mode)))


def ffn_masked(X, mask, W_gate, W_up, W_down_packed, *, mode="prefill", out=None, workspace=None,
               sort_tokens=False):
    """wide_ffn_masked.  X [T, d] bf16, mask [T, n] uint8, W_gate/W_up [F, d] bf16,
    W_down_packed [n, d, G] bf16 (see pack_kmajor).  Returns Y [T, d] bf16.
    sort_tokens: WIDE_FLAG_FFN_TOKEN_SORT."""
    for t, nm in ((X, "X"), (W_gate, "W_gate"), (W_up, "W_up"), (W_down_packed, "W_down_packed")):
        _dev(t, torch.bfloat16, nm)
    _dev(mask, torch.uint8, "mask")
    T, d = X.shape
    F = W_gate.shape[0]
    n = mask.shape[1]
    if mask.shape[0] != T or W_gate.shape != (F, d) or W_up.shape != (F, d):
        raise ValueError("shape mismatch")
    if W_down_packed.shape != (n, d, F // n):
        raise ValueError("W_down_packed must be [n_groups, d_model, d_ff / n_groups]")
    m = _mode(mode)
    ws_bytes = ffn_masked_workspace(T, d, F, n, m)
    ws = _workspace(ws_bytes, X.device, workspace)
    Y = out if out is not None else torch.empty((T, d), dtype=torch.bfloat16, device=X.device)
    st = lib().wide_ffn_masked(_ptr(X), _ptr(mask), _ptr(W_gate), _ptr(W_up), _ptr(W_down_packed),
                               T, d, F, n, m, _ptr(Y), _ptr(ws), ws.numel(),
                               WIDE_FLAG_FFN_TOKEN_SORT if sort_tokens else 0, _stream())
    _check("wide_ffn_masked", st)
    return Y


def ffn_masked_f32_workspace(T, d_model, d_ff, n_groups) -> int:
    return int(lib().wide_ffn_masked_f32_workspace(T, d_model, d_ff, n_groups))


def ffn_masked_f32(X, mask, W_gate, W_up, W_down, *, out=None, workspace=None):
    """wide_ffn_masked_f32: the masked FFN in fp32 throughout.  X [T, d] fp32, mask
    [T, n] uint8, W_gate/W_up/W_down [F, d] fp32 (W_down as is, not packed).
    Returns Y [T, d] fp32."""
    for t, nm in ((X, "X"), (W_gate, "W_gate"), (W_up, "W_up"), (W_down, "W_down")):
        _dev(t, torch.float32, nm)
    _dev(mask, torch.uint8, "mask")
    T, d = X.shape
    F = W_gate.shape[0]
    n = mask.shape[1]
    if mask.shape[0] != T or any(w.shape != (F, d) for w in (W_gate, W_up, W_down)):
        raise ValueError("shape mismatch")
    ws = _workspace(ffn_masked_f32_workspace(T, d, F, n), X.device, workspace)
    Y = out if out is not None else torch.empty((T, d), dtype=torch.float32, device=X.device)
    st = lib().wide_ffn_masked_f32(_ptr(X), _ptr(mask), _ptr(W_gate), _ptr(W_up), _ptr(W_down),
                                   T, d, F, n, _ptr(Y), _ptr(ws), ws.numel(), 0, _stream())
    _check("wide_ffn_masked_f32", st)
    return Y


NOALLOC_SCRATCH_BYTES = 16 << 20  # WIDE_NOALLOC_SCRATCH_BYTES


def ffn_masked_noalloc(X, mask, W_gate, W_up, W_down_packed, *, mode="prefill", out):
    """wide_ffn_masked_noalloc: ffn_masked with the library's fixed per-GPU scratch
    instead of a workspace; ``out`` (Y [T, d] bf16) is required, nothing is allocated.
    Calls that may overlap on one GPU race on the scratch."""
    for t, nm in ((X, "X"), (W_gate, "W_gate"), (W_up, "W_up"), (W_down_packed, "W_down_packed"),
                  (out, "out")):
        _dev(t, torch.bfloat16, nm)
    _dev(mask, torch.uint8, "mask")
    T, d = X.shape
    F = W_gate.shape[0]
    n = mask.shape[1]
    if mask.shape[0] != T or W_gate.shape != (F, d) or W_up.shape != (F, d) or out.shape != (T, d):
        raise ValueError("shape mismatch")
    if W_down_packed.shape != (n, d, F // n):
        raise ValueError("W_down_packed must be [n_groups, d_model, d_ff / n_groups]")
    st = lib().wide_ffn_masked_noalloc(_ptr(X), _ptr(mask), _ptr(W_gate), _ptr(W_up),
                                       _ptr(W_down_packed), T, d, F, n, _mode(mode), _ptr(out), 0,
                                       _stream())
    _check("wide_ffn_masked_noalloc", st)
    return out


# ---------------------------------------------------------------- attention

def _attn_cfg(n_q, n_kv, hd, theta):
    return WideAttnCfg(n_q, n_kv, hd, float(theta))


def attn_proj_masked_workspace(T, d_model, n_q, n_kv, head_dim=128, rope_theta=0.0,
                               mode="prefill", kv_cap=0) -> int:
    cfg = _attn_cfg(n_q, n_kv, head_dim, rope_theta)
    return int(lib().wide_attn_proj_masked_workspace(T, d_model, C.byref(cfg), _mode(mode), kv_cap))


def attn_proj_masked(X, mask, Wq, Wk, Wv, Wo_packed, *, n_q, n_kv, head_dim=128, rope_theta=0.0,
                     mode="prefill", K_cache=None, V_cache=None, kv_len=0, out=None,
                     workspace=None):
    """wide_attn_proj_masked.  Returns Y [T, d] bf16 (decode also writes the caches)."""
    for t, nm in ((X, "X"), (Wq, "Wq"), (Wk, "Wk"), (Wv, "Wv"), (Wo_packed, "Wo_packed")):
        _dev(t, torch.bfloat16, nm)
    _dev(mask, torch.uint8, "mask")
    m = _mode(mode)
    T, d = X.shape
    kv_cap = 0
    if m == WIDE_DECODE:
        _dev(K_cache, torch.bfloat16, "K_cache")
        _dev(V_cache, torch.bfloat16, "V_cache")
        kv_cap = K_cache.shape[2]
    cfg = _attn_cfg(n_q, n_kv, head_dim, rope_theta)
    ws_bytes = int(lib().wide_attn_proj_masked_workspace(T, d, C.byref(cfg), m, kv_cap))
    ws = _workspace(ws_bytes, X.device, workspace)
    Y = out if out is not None else torch.empty((T, d), dtype=torch.bfloat16, device=X.device)
    st = lib().wide_attn_proj_masked(_ptr(X), _ptr(mask), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                                     _ptr(Wo_packed), T, d, C.byref(cfg), m, _ptr(K_cache),
                                     _ptr(V_cache), kv_len, kv_cap, _ptr(Y), _ptr(ws), ws.numel(),
                                     0, _stream())
    _check("wide_attn_proj_masked", st)
    return Y


def attn_decode_masked_cache(X, mask, Wq, Wk, Wv, Wo_packed, *, n_q, n_kv, K_cache, V_cache,
                             kv_len, pos, head_dim=128, rope_theta=0.0, out=None, workspace=None):
    """wide_attn_decode_masked_cache: one decode step over per-(sequence, group) cache
    lengths kv_len (int32 [B, n_kv] device tensor, not modified: advance it by the mask
    after the call).  Returns Y [B, d] bf16; writes the kept pairs' new K/V."""
    for t, nm in ((X, "X"), (Wq, "Wq"), (Wk, "Wk"), (Wv, "Wv"), (Wo_packed, "Wo_packed"),
                  (K_cache, "K_cache"), (V_cache, "V_cache")):
        _dev(t, torch.bfloat16, nm)
    _dev(mask, torch.uint8, "mask")
    _dev(kv_len, torch.int32, "kv_len")
    B, d = X.shape
    kv_cap = K_cache.shape[2]
    cfg = _attn_cfg(n_q, n_kv, head_dim, rope_theta)
    ws_bytes = int(lib().wide_attn_proj_masked_workspace(B, d, C.byref(cfg), WIDE_DECODE, kv_cap))
    ws = _workspace(ws_bytes, X.device, workspace)
    Y = out if out is not None else torch.empty((B, d), dtype=torch.bfloat16, device=X.device)
    st = lib().wide_attn_decode_masked_cache(_ptr(X), _ptr(mask), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                                             _ptr(Wo_packed), B, d, C.byref(cfg), _ptr(K_cache),
                                             _ptr(V_cache), kv_cap, _ptr(kv_len), int(pos), _ptr(Y),
                                             _ptr(ws), ws.numel(), 0, _stream())
    _check("wide_attn_decode_masked_cache", st)
    return Y


def attn_decode_masked_paged(X, mask, Wq, Wk, Wv, Wo_packed, *, n_q, n_kv, K_pool, V_pool,
                             page_table, kv_len, pos, head_dim=128, rope_theta=0.0, out=None,
                             workspace=None):
    """wide_attn_decode_masked_paged: attn_decode_masked_cache over a paged cache.
    K_pool, V_pool [n_pages, page_size, head_dim] bf16; page_table [B, n_kv, max_pages]
    int32 (slot s of pair (b, g) is row s % page_size of page page_table[b, g,
    s // page_size]); kv_len int32 [B, n_kv], not modified.  Returns Y [B, d] bf16;
    writes the kept pairs' new K/V into their pages."""
    for t, nm in ((X, "X"), (Wq, "Wq"), (Wk, "Wk"), (Wv, "Wv"), (Wo_packed, "Wo_packed"),
                  (K_pool, "K_pool"), (V_pool, "V_pool")):
        _dev(t, torch.bfloat16, nm)
    _dev(mask, torch.uint8, "mask")
    _dev(kv_len, torch.int32, "kv_len")
    _dev(page_table, torch.int32, "page_table")
    B, d = X.shape
    n_pages, page_size = K_pool.shape[0], K_pool.shape[1]
    if tuple(V_pool.shape) != tuple(K_pool.shape) or page_table.dim() != 3:
        raise ValueError("K_pool and V_pool must match; page_table must be [B, n_kv, max_pages]")
    max_pages = page_table.shape[2]
    cfg = _attn_cfg(n_q, n_kv, head_dim, rope_theta)
    ws_bytes = int(lib().wide_attn_proj_masked_workspace(B, d, C.byref(cfg), WIDE_DECODE,
                                                         max_pages * page_size))
    ws = _workspace(ws_bytes, X.device, workspace)
    Y = out if out is not None else torch.empty((B, d), dtype=torch.bfloat16, device=X.device)
    st = lib().wide_attn_decode_masked_paged(_ptr(X), _ptr(mask), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                                             _ptr(Wo_packed), B, d, C.byref(cfg), _ptr(K_pool),
                                             _ptr(V_pool), n_pages, page_size, _ptr(page_table),
                                             max_pages, _ptr(kv_len), int(pos), _ptr(Y), _ptr(ws),
                                             ws.numel(), 0, _stream())
    _check("wide_attn_decode_masked_paged", st)
    return Y


# -------------------------------------------------------------------- layer

def _layer_cfg(d, F, n_ffn, n_q, n_kv, hd, theta, eps):
    return WideLayerCfg(d, F, n_ffn, _attn_cfg(n_q, n_kv, hd, theta), float(eps))


def layer_masked_workspace(T, d_model, d_ff, n_ffn, n_q, n_kv, head_dim=128, rope_theta=500000.0,
                           eps=1e-5, mode="prefill", kv_cap=0) -> int:
    cfg = _layer_cfg(d_model, d_ff, n_ffn, n_q, n_kv, head_dim, rope_theta, eps)
    return int(lib().wide_layer_masked_workspace(T, C.byref(cfg), _mode(mode), kv_cap))


def layer_masked(X, attn_mask, ffn_mask, W: dict, *, n_q, n_kv, head_dim=128,
                 rope_theta=500000.0, eps=1e-5, mode="prefill", K_cache=None, V_cache=None,
                 kv_len=0, out=None, workspace=None, sort_ffn_tokens=False):
    """wide_layer_masked.  W: rms1, rms2 [d]; Wq, Wk, Wv; Wo_packed; W_gate, W_up;
    W_down_packed (all bf16 device tensors).  sort_ffn_tokens: WIDE_FLAG_FFN_TOKEN_SORT."""
    _dev(X, torch.bfloat16, "X")
    _dev(attn_mask, torch.uint8, "attn_mask")
    _dev(ffn_mask, torch.uint8, "ffn_mask")
    keys = ("rms1", "Wq", "Wk", "Wv", "Wo_packed", "rms2", "W_gate", "W_up", "W_down_packed")
    for k in keys:
        _dev(W[k], torch.bfloat16, k)
    m = _mode(mode)
    T, d = X.shape
    F = W["W_gate"].shape[0]
    n_ffn = ffn_mask.shape[1]
    kv_cap = 0
    if m == WIDE_DECODE:
        _dev(K_cache, torch.bfloat16, "K_cache")
        _dev(V_cache, torch.bfloat16, "V_cache")
        kv_cap = K_cache.shape[2]
    cfg = _layer_cfg(d, F, n_ffn, n_q, n_kv, head_dim, rope_theta, eps)
    wts = WideLayerWeights(*[W[k].data_ptr() for k in keys])
    ws_bytes = int(lib().wide_layer_masked_workspace(T, C.byref(cfg), m, kv_cap))
    ws = _workspace(ws_bytes, X.device, workspace)
    Y = out if out is not None else torch.empty((T, d), dtype=torch.bfloat16, device=X.device)
    st = lib().wide_layer_masked(_ptr(X), _ptr(attn_mask), _ptr(ffn_mask), C.byref(wts),
                                 C.byref(cfg), T, m, _ptr(K_cache), _ptr(V_cache), kv_len, kv_cap,
                                 _ptr(Y), _ptr(ws), ws.numel(),
                                 WIDE_FLAG_FFN_TOKEN_SORT if sort_ffn_tokens else 0, _stream())
    _check("wide_layer_masked", st)
    return Y


_LAYER_KEYS = ("rms1", "Wq", "Wk", "Wv", "Wo_packed", "rms2", "W_gate", "W_up", "W_down_packed")


def _layer_weights(W: dict):
    for k in _LAYER_KEYS:
        _dev(W[k], torch.bfloat16, k)
    return WideLayerWeights(*[W[k].data_ptr() for k in _LAYER_KEYS])


def layer_masked_routed(X, R_attn_packed, k_attn, R_ffn_packed, k_ffn, W: dict, *, n_q, n_kv,
                        n_ffn, head_dim=128, rope_theta=500000.0, eps=1e-5, mode="prefill",
                        K_cache=None, V_cache=None, kv_len=0, out=None, attn_mask=None,
                        ffn_mask=None, workspace=None, sort_ffn_tokens=False):
    """wide_layer_masked_routed: the layer with masks chosen on the GPU by two linear
    routers on X (R_*_packed from pack_router).  Returns (Y, attn_mask, ffn_mask).
    sort_ffn_tokens: WIDE_FLAG_FFN_TOKEN_SORT."""
    _dev(X, torch.bfloat16, "X")
    _dev(R_attn_packed, torch.bfloat16, "R_attn_packed")
    _dev(R_ffn_packed, torch.bfloat16, "R_ffn_packed")
    m = _mode(mode)
    T, d = X.shape
    F = W["W_gate"].shape[0]
    kv_cap = 0
    if m == WIDE_DECODE:
        _dev(K_cache, torch.bfloat16, "K_cache")
        _dev(V_cache, torch.bfloat16, "V_cache")
        kv_cap = K_cache.shape[2]
    cfg = _layer_cfg(d, F, n_ffn, n_q, n_kv, head_dim, rope_theta, eps)
    wts = _layer_weights(W)
    rt = WideLayerRouter(R_attn_packed.data_ptr(), R_ffn_packed.data_ptr(), int(k_attn),
                         int(k_ffn))
    ws_bytes = int(lib().wide_layer_masked_workspace(T, C.byref(cfg), m, kv_cap))
    ws = _workspace(ws_bytes, X.device, workspace)
    Y = out if out is not None else torch.empty((T, d), dtype=torch.bfloat16, device=X.device)
    am = attn_mask if attn_mask is not None else torch.empty((T, n_kv), dtype=torch.uint8,
                                                             device=X.device)
    fm = ffn_mask if ffn_mask is not None else torch.empty((T, n_ffn), dtype=torch.uint8,
                                                           device=X.device)
    st = lib().wide_layer_masked_routed(_ptr(X), C.byref(rt), C.byref(wts), C.byref(cfg), T, m,
                                        _ptr(K_cache), _ptr(V_cache), kv_len, kv_cap, _ptr(am),
                                        _ptr(fm), _ptr(Y), _ptr(ws), ws.numel(),
                                        WIDE_FLAG_FFN_TOKEN_SORT if sort_ffn_tokens else 0,
                                        _stream())
    _check("wide_layer_masked_routed", st)
    return Y, am, fm


def layer_decode_masked_cache(X, attn_mask, ffn_mask, W: dict, *, n_q, n_kv, K_cache, V_cache,
                              kv_len, pos, head_dim=128, rope_theta=500000.0, eps=1e-5, out=None,
                              workspace=None):
    """wide_layer_decode_masked_cache: one layer decode step over per-(sequence, group)
    cache lengths kv_len (int32 [B, n_kv], not modified).  Returns Y [B, d]."""
    _dev(X, torch.bfloat16, "X")
    _dev(attn_mask, torch.uint8, "attn_mask")
    _dev(ffn_mask, torch.uint8, "ffn_mask")
    _dev(K_cache, torch.bfloat16, "K_cache")
    _dev(V_cache, torch.bfloat16, "V_cache")
    _dev(kv_len, torch.int32, "kv_len")
    B, d = X.shape
    F = W["W_gate"].shape[0]
    n_ffn = ffn_mask.shape[1]
    kv_cap = K_cache.shape[2]
    cfg = _layer_cfg(d, F, n_ffn, n_q, n_kv, head_dim, rope_theta, eps)
    wts = _layer_weights(W)
    ws_bytes = int(lib().wide_layer_masked_workspace(B, C.byref(cfg), WIDE_DECODE, kv_cap))
    ws = _workspace(ws_bytes, X.device, workspace)
    Y = out if out is not None else torch.empty((B, d), dtype=torch.bfloat16, device=X.device)
    st = lib().wide_layer_decode_masked_cache(_ptr(X), _ptr(attn_mask), _ptr(ffn_mask),
                                              C.byref(wts), C.byref(cfg), B, _ptr(K_cache),
                                              _ptr(V_cache), kv_cap, _ptr(kv_len), int(pos),
                                              _ptr(Y), _ptr(ws), ws.numel(), 0, _stream())
    _check("wide_layer_decode_masked_cache", st)
    return Y


def layer_decode_masked_paged(X, attn_mask, ffn_mask, W: dict, *, n_q, n_kv, K_pool, V_pool,
                              page_table, kv_len, pos, head_dim=128, rope_theta=500000.0,
                              eps=1e-5, out=None, workspace=None):
    """wide_layer_decode_masked_paged: layer_decode_masked_cache over a paged pool
    (K_pool, V_pool [n_pages, page_size, head_dim]; page_table [B, n_kv, max_pages])."""
    _dev(X, torch.bfloat16, "X")
    _dev(attn_mask, torch.uint8, "attn_mask")
    _dev(ffn_mask, torch.uint8, "ffn_mask")
    _dev(K_pool, torch.bfloat16, "K_pool")
    _dev(V_pool, torch.bfloat16, "V_pool")
    _dev(kv_len, torch.int32, "kv_len")
    _dev(page_table, torch.int32, "page_table")
    B, d = X.shape
    F = W["W_gate"].shape[0]
    n_ffn = ffn_mask.shape[1]
    n_pages, page_size = K_pool.shape[0], K_pool.shape[1]
    if tuple(V_pool.shape) != tuple(K_pool.shape) or page_table.dim() != 3:
        raise ValueError("K_pool and V_pool must match; page_table must be [B, n_kv, max_pages]")
    max_pages = page_table.shape[2]
    cfg = _layer_cfg(d, F, n_ffn, n_q, n_kv, head_dim, rope_theta, eps)
    wts = _layer_weights(W)
    ws_bytes = int(lib().wide_layer_masked_workspace(B, C.byref(cfg), WIDE_DECODE,
                                                     max_pages * page_size))
    ws = _workspace(ws_bytes, X.device, workspace)
    Y = out if out is not None else torch.empty((B, d), dtype=torch.bfloat16, device=X.device)
    st = lib().wide_layer_decode_masked_paged(_ptr(X), _ptr(attn_mask), _ptr(ffn_mask),
                                              C.byref(wts), C.byref(cfg), B, _ptr(K_pool),
                                              _ptr(V_pool), n_pages, page_size, _ptr(page_table),
                                              max_pages, _ptr(kv_len), int(pos), _ptr(Y),
                                              _ptr(ws), ws.numel(), 0, _stream())
    _check("wide_layer_decode_masked_paged", st)
    return Y
