"""GPU parity of wide_attn_proj_masked against the oracle (reading: a kept token
attends causally to the tokens that also keep its group; dropped groups give 0).
Bar: max|err| / max|ref| <= 1e-2; outputs NaN-filled before the call."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import attn_masked
from synth.workloads import attn_case, attn_prefill_8b
from tests._gpu import TOL, bf16, dev, host, log, nan_bf16, needs_gpu, rel_err, u8


def _gpu_attn(c, theta, **kw):
    m = c["meta"]
    T, d = c["X"].shape
    Y = nan_bf16((T, d))
    wide.attn_proj_masked(bf16(c["X"]), u8(c["mask"]), bf16(c["Wq"]), bf16(c["Wk"]), bf16(c["Wv"]),
                          wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]), n_q=m["n_q"], n_kv=m["n_kv"],
                          head_dim=128, rope_theta=theta, out=Y, **kw)
    torch.cuda.synchronize()
    return host(Y)


def _oracle(c, theta, rows=None):
    m = c["meta"]
    return attn_masked(c["X"], c["mask"], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                       n_kv=m["n_kv"], head_dim=128, rope_theta=theta, rows=rows)


SHAPES = [
    # T, d, n_q, n_kv, keep, kind, theta
    (300, 256, 8, 2, 0.5, "topk", 0.0),
    (513, 512, 16, 4, 0.5, "bernoulli", 500000.0),
    (257, 256, 12, 4, 0.5, "topk", 10000.0),      # r = 3
    (200, 256, 16, 2, 0.75, "bernoulli", 0.0),    # r = 8
    (129, 384, 8, 8, 0.25, "clustered", 500000.0),  # r = 1
    (1, 256, 8, 2, 0.5, "ones", 500000.0),
    (333, 256, 8, 2, 1.0, "ones", 500000.0),
    (190, 256, 8, 2, 0.0, "zeros", 0.0),
    (1100, 256, 8, 8, 0.5, "topk", 500000.0),
    # many groups: fewer bins per group than tile pairs, so a bin takes 3 or more
    # query tiles in snake order (8 bins of 32 tiles; 4 bins; 16 bins of 35 tiles)
    (2048, 256, 32, 32, 1.0, "ones", 500000.0),
    (1500, 256, 64, 64, 0.75, "bernoulli", 0.0),
    (2200, 256, 64, 16, 1.0, "ones", 10000.0),
]


@needs_gpu
@pytest.mark.parametrize("T,d,n_q,n_kv,keep,kind,theta", SHAPES)
def test_attn_prefill_shapes(T, d, n_q, n_kv, keep, kind, theta):
    dev()
    log(f"attn prefill T={T} d={d} n_q={n_q} n_kv={n_kv} keep={keep} {kind} theta={theta}")
    c = attn_case(f"attn_{T}_{d}_{n_q}_{n_kv}_{kind}", T, d, n_q, n_kv, 128, keep, kind)
    got = _gpu_attn(c, theta)
    ref = _oracle(c, theta)
    if kind == "zeros":
        assert np.all(got == 0.0)
    assert rel_err(got, ref) <= TOL


@needs_gpu
def test_attn_prefill_llama31_8b_full():
    """Llama-3.1-8B attention prefill: T=2048, d=4096, 32 query / 8 KV heads,
    keep 4 of 8 groups, no RoPE; every output row checked."""
    dev()
    log("attn prefill 8B full T=2048")
    c = attn_prefill_8b()
    got = _gpu_attn(c, 0.0)
    ref = _oracle(c, 0.0)
    assert rel_err(got, ref) <= TOL
