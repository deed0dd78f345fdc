"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every entry point include/wide.h declares, answers
workspace queries and rejects bad arguments before touching the GPU.
"""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wide.h")


@pytest.fixture(scope="module")
def L():
    from sparse_wide_mask_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libwide.so not built")
    return binding.lib()


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const char\*|int|size_t|void)\s+(wide_\w+)\(", src, re.M)))


def test_header_declares_the_contract():
    names = declared()
    for fn in ("wide_mask_reorder", "wide_ffn_masked", "wide_attn_proj_masked", "wide_layer_masked"):
        assert fn in names


def test_every_declared_symbol_is_exported(L):
    for name in declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    assert L.wide_status_string(0) == b"ok"
    assert L.wide_status_string(3) == b"workspace too small"
    assert L.wide_version() >= 1


def test_ffn_workspace_queries(L):
    from sparse_wide_mask_amd import binding as b
    ws = b.ffn_masked_workspace(4096, 3072, 8192, 64)
    assert ws >= 4096 * 8192 * 2                      # H is held in the workspace
    assert b.ffn_masked_workspace(64, 256, 1000, 16) == 0   # d_ff % n != 0 -> invalid -> 0
    assert b.ffn_masked_workspace(64, 256, 16 * 96, 16) == 0  # G = 96: unsupported -> 0
    assert b.ffn_masked_workspace(64, 256, 16 * 16, 16) == 0  # G = 16: unsupported -> 0
    assert b.ffn_masked_workspace(64, 256, 16 * 32, 16) > 0   # G = 32: supported


def test_validation_before_any_launch(L):
    # NULL pointers and bad shapes are rejected on the host: no GPU is touched.
    z = C.c_void_p(0)
    assert L.wide_mask_reorder(z, 10, 4, 4, z, z, z, z, z, z, z) == 1
    assert L.wide_mask_reorder(z, 10, 0, 4, z, z, z, z, z, z, z) == 1
    assert L.wide_mask_reorder(z, 10, 300, 4, z, z, z, z, z, z, z) == 2
    assert L.wide_mask_reorder(z, 0, 4, 4, z, z, z, z, z, z, z) == 0     # T == 0: no-op
    assert L.wide_ffn_masked(z, z, z, z, z, 8, 256, 1000, 16, 0, z, z, 0, 0, z) == 1
    assert L.wide_ffn_masked(z, z, z, z, z, 8, 256, 1024, 16, 0, z, z, 0, 0, z) == 1
    assert L.wide_ffn_masked(z, z, z, z, z, 8, 200, 1024, 16, 0, z, z, 0, 0, z) == 2
    assert L.wide_ffn_masked(z, z, z, z, z, 8, 256, 1024, 16, 7, z, z, 0, 0, z) == 1
    assert L.wide_ffn_masked(z, z, z, z, z, 0, 256, 1024, 16, 0, z, z, 0, 0, z) == 0
    # flags: the FFN token sort bit is taken, every other bit rejected
    assert L.wide_ffn_masked(z, z, z, z, z, 0, 256, 1024, 16, 0, z, z, 0, 2, z) == 0
    assert L.wide_ffn_masked(z, z, z, z, z, 0, 256, 1024, 16, 0, z, z, 0, 1, z) == 1
    assert L.wide_ffn_masked(z, z, z, z, z, 0, 256, 1024, 16, 0, z, z, 0, 6, z) == 1
    assert L.wide_pack_kmajor(z, 4, 64, 256, z, z) == 1
    buf = C.c_void_p(16)  # aligned, never dereferenced: the shape is rejected first
    other = C.c_void_p(32)
    assert L.wide_pack_kmajor(buf, 4, 16, 256, other, z) == 2   # G = 16: unsupported


def test_ffn_f32_validation_and_workspace(L):
    from sparse_wide_mask_amd import binding as b
    z = C.c_void_p(0)
    assert b.ffn_masked_f32_workspace(64, 256, 1024, 16) >= 64 * 1024 * 4   # H in fp32
    assert b.ffn_masked_f32_workspace(37, 100, 16 * 24, 16) >= 37 * 384 * 4  # any G and d
    assert b.ffn_masked_f32_workspace(64, 256, 1000, 16) == 0   # d_ff % n != 0
    assert b.ffn_masked_f32_workspace(64, 256, 1200, 300) == 0  # too many groups
    f = L.wide_ffn_masked_f32
    assert f(z, z, z, z, z, 8, 256, 1000, 16, z, z, 0, 0, z) == 1   # d_ff % n != 0
    assert f(z, z, z, z, z, 8, 256, 1200, 300, z, z, 0, 0, z) == 2  # n > 256
    assert f(z, z, z, z, z, 8, 256, 1024, 16, z, z, 0, 0, z) == 1   # NULL pointers
    assert f(z, z, z, z, z, 8, 256, 1024, 16, z, z, 0, 1, z) == 1   # flags != 0
    assert f(z, z, z, z, z, 0, 256, 1024, 16, z, z, 0, 0, z) == 0   # T == 0: no-op
    p = [C.c_void_p(16 * (i + 1)) for i in range(7)]  # aligned, never dereferenced
    assert f(*p[:5], 8, 256, 1024, 16, p[5], p[6], 16, 0, z) == 3   # workspace too small


def test_router_validation_before_any_launch(L):
    z = C.c_void_p(0)
    assert L.wide_router_topk(z, z, 8, 256, 16, 8, z, z, z, z) == 1     # NULL X / R / mask
    assert L.wide_router_topk(z, z, 8, 256, 16, 17, z, z, z, z) == 1    # k > n_groups
    assert L.wide_router_topk(z, z, 8, 256, 16, -1, z, z, z, z) == 1
    assert L.wide_router_topk(z, z, 8, 256, 0, 0, z, z, z, z) == 1      # no groups
    assert L.wide_router_topk(z, z, 8, 200, 16, 8, z, z, z, z) == 2     # d_model % 64
    assert L.wide_router_topk(z, z, 8, 256, 257, 8, z, z, z, z) == 2    # too many groups
    assert L.wide_router_topk(z, z, 0, 256, 16, 8, z, z, z, z) == 0     # T == 0: no-op


def test_masked_cache_decode_validation_before_any_launch(L):
    from sparse_wide_mask_amd import binding as b
    z = C.c_void_p(0)
    cfg = b.WideAttnCfg(32, 8, 128, 0.0)
    args = lambda B, d, cfgp, cap, pos: (z, z, z, z, z, z, B, d, cfgp, z, z, cap, z, pos, z, z, 0, 0, z)
    assert L.wide_attn_decode_masked_cache(*args(4, 4096, None, 10, 0)) == 1       # no cfg
    assert L.wide_attn_decode_masked_cache(*args(4, 4096, C.byref(cfg), 10, -1)) == 1  # pos < 0
    assert L.wide_attn_decode_masked_cache(*args(4, 4096, C.byref(cfg), 0, 0)) == 1   # no slots
    assert L.wide_attn_decode_masked_cache(*args(65, 4096, C.byref(cfg), 10, 0)) == 2  # batch > 64
    assert L.wide_attn_decode_masked_cache(*args(4, 4096, C.byref(cfg), 10, 0)) == 1   # NULL caches


def test_paged_decode_validation_before_any_launch(L):
    from sparse_wide_mask_amd import binding as b
    z = C.c_void_p(0)
    k, v = C.c_void_p(16), C.c_void_p(32)  # aligned, never dereferenced
    cfg = b.WideAttnCfg(32, 8, 128, 0.0)

    def call(B=4, cfgp=None, pages=8, ps=16, maxp=4, pos=0, kp=k, vp=v):
        return L.wide_attn_decode_masked_paged(z, z, z, z, z, z, B, 4096, cfgp or C.byref(cfg),
                                               kp, vp, pages, ps, z, maxp, z, pos, z, z, 0, 0, z)
    assert call(pos=-1) == 1                      # pos < 0
    assert call(ps=8) == 1                        # page below 16 slots
    assert call(ps=48) == 1                       # not a power of two
    assert call(pages=0) == 1                     # empty pool
    assert call(maxp=0) == 1                      # no pages per pair
    assert call(kp=z) == 1                        # NULL pool
    assert call(vp=k) == 1                        # K and V pools alias
    assert call(B=65) == 2                        # batch > 64
    assert call(pages=1 << 20, ps=64) == 2        # pool past 2 GiB
    assert call(maxp=1 << 20, ps=64) == 2         # a pair's slots past 2 GiB
    assert call(B=0) == 0                         # empty batch: no-op
    assert call() == 1                            # NULL X, table, lengths


def test_pack_router_validation(L):
    z = C.c_void_p(0)
    assert L.wide_pack_router(z, 16, 256, z, z) == 1
    assert L.wide_pack_router(z, 300, 256, z, z) == 2
    assert L.wide_pack_router(z, 16, 200, z, z) == 2
