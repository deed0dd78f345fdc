"""GPU parity of wide_ffn_masked_f32, the masked SwiGLU FFN computed in fp32 throughout
(fp32 inputs as drawn, no bf16 rounding), against the fp64 oracle.

Bar: max|err| / max|ref| <= 1e-5.  Each output is a chain of fp32 fused multiply-adds
over d_model (up) and d_ff (down) terms; the rounding of such a chain grows like
sqrt(K) * 2^-24 relative to the sum's scale (1.9e-6 at K = 1024), and the tiny
configuration's own fp32 oracle (NumPy, blocked sums) lands within the same order of
the fp64 result.  A wrong mask, group or index moves outputs by their own magnitude.
Dropped groups and tokens that keep none give exact zeros."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import ffn_masked
from synth import normal
from synth.workloads import make_mask
from tests._gpu import dev, host, log, nan_f32, needs_gpu, rel_err, u8

TOL32 = 1e-5


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev())


def _case(cfg, T, d, F, n, keep, kind):
    """Raw fp32 draws (X ~ N(0,1), weights ~ N(0, 0.02)) and a mask."""
    X = normal(cfg, "X", (T, d), round_bf16=False)
    W = {k: normal(cfg, k, (F, d), 0.02, round_bf16=False) for k in ("W_gate", "W_up", "W_down")}
    return dict(X=X, mask=make_mask(cfg, T, n, keep, kind, X), **W)


def _gpu(c):
    T, d = c["X"].shape
    Y = nan_f32((T, d))
    wide.ffn_masked_f32(_f32(c["X"]), u8(c["mask"]), _f32(c["W_gate"]), _f32(c["W_up"]),
                        _f32(c["W_down"]), out=Y)
    torch.cuda.synchronize()
    return host(Y)


def _check(c, label):
    got = _gpu(c)
    ref = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"])
    e = rel_err(got, ref)
    e32 = rel_err(ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"],
                             dtype=np.float32), ref)
    log(f"{label}: fp32 GPU vs fp64 oracle {e:.2e} (fp32 oracle vs fp64 {e32:.2e})")
    assert e <= TOL32
    none = ~np.any(c["mask"] != 0, axis=1)  # tokens that keep no group: exact zeros
    assert np.all(got[none] == 0.0)
    return got


@needs_gpu
def test_tiny_configuration_in_fp32():
    """The tiny configuration as declared: fp32, d 256, d_ff 1024 in 16 groups of 64,
    64 tokens keeping 8 of 16 groups by top-k of N(0,1) logits."""
    dev()
    from synth.workloads import tiny_ffn
    c0 = tiny_ffn()
    c = {k: normal("tiny_ffn", k, c0[k].shape, 1.0 if k == "X" else 0.02, round_bf16=False)
         for k in ("X", "W_gate", "W_up", "W_down")}
    c["mask"] = c0["mask"]
    assert (c["mask"] != 0).sum(axis=1).tolist() == [8] * 64
    _check(c, "tiny fp32 configuration")


@needs_gpu
@pytest.mark.parametrize("T,d,F,n,keep,kind", [
    (37, 100, 384, 16, 0.5, "bernoulli"),     # G = 24, d not a multiple of 64, ragged T
    (130, 320, 1536, 12, 0.5, "topk"),        # G = 128
    (5, 64, 256, 256, 0.5, "bernoulli"),      # groups of one channel, 256 groups
    (200, 257, 1000, 8, 0.25, "clustered"),   # G = 125, odd d
    (64, 256, 1024, 16, 1.0, "ones"),         # all kept: the dense FFN
    (2000, 512, 2048, 32, 0.5, "topk"),       # many tiles
])
def test_ffn_f32_shapes(T, d, F, n, keep, kind):
    dev()
    _check(_case(f"ffn32_{T}_{d}_{F}_{n}_{kind}", T, d, F, n, keep, kind),
           f"ffn fp32 T={T} d={d} F={F} n={n} {kind}")


@needs_gpu
def test_ffn_f32_zero_masks_and_repeat():
    """All-zero masks give exact zeros; a repeated call gives the same bits."""
    dev()
    c = _case("ffn32_zero", 50, 128, 512, 8, 0.0, "zeros")
    assert np.all(_gpu(c) == 0.0)
    c = _case("ffn32_rep", 90, 192, 768, 12, 0.5, "topk")
    a, b = _gpu(c), _gpu(c)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
