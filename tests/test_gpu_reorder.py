"""GPU parity of wide_mask_reorder against the oracle: bit-exact on every output."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import mask_reorder
from synth.workloads import make_mask
from tests._gpu import dev, host, log, needs_gpu, u8

KEYS = ("packed", "group_count", "group_perm", "group_rank", "tile_count", "tile_groups")


def _run(m, tile_m):
    out = wide.mask_reorder(u8(m), tile_m)
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in out.items()}
    ref = mask_reorder(m, tile_m)
    for k in KEYS:
        g = got[k].view(np.uint64) if k == "packed" else got[k]
        assert np.array_equal(g.astype(np.uint64) if k == "packed" else g,
                              ref[k].astype(g.dtype)), f"{k} differs (T={m.shape[0]}, n={m.shape[1]})"


CASES = [
    (1, 1, 1, "bernoulli", 0.5), (5, 3, 2, "bernoulli", 0.5), (63, 8, 64, "topk", 0.5),
    (64, 64, 64, "bernoulli", 0.3), (65, 65, 64, "bernoulli", 0.7), (1000, 112, 256, "topk", 0.5),
    (1025, 16, 128, "clustered", 0.25), (2048, 8, 256, "topk", 0.5), (3000, 129, 100, "bernoulli", 0.5),
    (4096, 64, 256, "bernoulli", 0.5), (777, 256, 1024, "bernoulli", 0.9), (300, 7, 1, "ones", 1.0),
    (300, 7, 33, "zeros", 0.0),
]


@needs_gpu
@pytest.mark.parametrize("T,n,tile_m,kind,keep", CASES)
def test_reorder_bit_exact(T, n, tile_m, kind, keep):
    dev()
    log(f"reorder T={T} n={n} tile_m={tile_m} {kind}")
    m = make_mask(f"reorder_{T}_{n}", T, n, keep, kind)
    # nonzero bytes other than 1 must also count as keep
    m = m * np.random.default_rng(T).integers(1, 256, m.shape).astype(np.uint8)
    _run(m, tile_m)


@needs_gpu
@pytest.mark.parametrize("T,n,kind", [(1, 1, "bernoulli"), (63, 8, "topk"), (1000, 8, "topk"),
                                      (4097, 4, "clustered"), (3000, 129, "bernoulli"),
                                      (8192, 8, "bernoulli"), (65536, 8, "topk")])
def test_reorder_without_unions_bit_exact(T, n, kind):
    """Null tile outputs: grouping and packing in one launch, the group work-groups
    reading the mask bytes; packed words, counts, permutations and ranks bit-exact."""
    dev()
    log(f"reorder without unions T={T} n={n} {kind}")
    m = make_mask(f"reorder_nu_{T}_{n}", T, n, 0.5, kind)
    m = m * np.random.default_rng(T + 1).integers(1, 256, m.shape).astype(np.uint8)
    out = wide.mask_reorder(u8(m), 256, unions=False)
    torch.cuda.synchronize()
    assert set(out) == {"packed", "group_count", "group_perm", "group_rank"}
    ref = mask_reorder(m, 256)
    assert np.array_equal(host(out["packed"]).view(np.uint64), ref["packed"].astype(np.uint64))
    for k in ("group_count", "group_perm", "group_rank"):
        assert np.array_equal(host(out[k]), ref[k]), k


@needs_gpu
@pytest.mark.parametrize("T,n", [(8192, 112), (8192, 8), (65536, 8), (32768, 160)])
def test_reorder_full_size(T, n):
    """The layer's mask sizes (8192 tokens x 112 FFN / 8 attention groups), the
    maximum token count, and a mask of more than 4 MB (packed by a launch of its own
    before the other roles); the oracle checks group 0..n-1 exactly."""
    dev()
    log(f"reorder full T={T} n={n}")
    m = make_mask(f"reorder_full_{T}_{n}", T, n, 0.5, "topk")
    _run(m, 256)


@needs_gpu
def test_reorder_repeat_is_deterministic():
    dev()
    m = u8(make_mask("reorder_det", 5000, 64, 0.5, "bernoulli"))
    a = {k: host(v) for k, v in wide.mask_reorder(m, 256).items()}
    b = {k: host(v) for k, v in wide.mask_reorder(m, 256).items()}
    for k in KEYS:
        assert np.array_equal(a[k], b[k])
