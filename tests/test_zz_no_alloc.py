"""The allocation-free FFN entry point, wide_ffn_masked_noalloc, called through the C ABI:
its output equals wide_ffn_masked's (same kernels, bit for bit) and the oracle's, on
two calls in a row that share the library's per-GPU scratch, the second one smaller.
Sizes over the scratch are rejected on the host."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import ffn_masked
from sparse_wide_mask_amd.binding import WIDE_EWORKSPACE, WideError
from synth.workloads import ffn_case, ffn_decode_8b
from tests._gpu import TOL, bf16, dev, host, log, nan_bf16, needs_gpu, rel_err, u8


def _args(c):
    n = c["mask"].shape[1]
    return (bf16(c["X"]), u8(c["mask"]), bf16(c["W_gate"]), bf16(c["W_up"]),
            wide.pack_kmajor(bf16(c["W_down"]), n))


@needs_gpu
def test_noalloc_matches_workspace_entry_point():
    dev()
    cases = [
        # first call: decode batch 64 at the Llama-3.1-8B FFN shape (about 10 MB of scratch)
        (ffn_decode_8b(64), "decode"),
        # second call, right after it: a smaller prefill with ragged tiles
        (ffn_case("ffn_noalloc_small", 300, 512, 2048, 16, 0.5, "bernoulli"), "prefill"),
    ]
    args = [_args(c) for c, _ in cases]
    outs = [nan_bf16(c["X"].shape) for c, _ in cases]
    torch.cuda.synchronize()
    for (c, mode), a, Y in zip(cases, args, outs):
        log(f"noalloc ffn {mode} T={c['X'].shape[0]} d={c['X'].shape[1]}")
        wide.ffn_masked_noalloc(*a, mode=mode, out=Y)
    torch.cuda.synchronize()
    for (c, mode), a, Y in zip(cases, args, outs):
        Yw = wide.ffn_masked(*a, mode=mode, out=nan_bf16(c["X"].shape))
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Yw.view(torch.int16)), mode
        ref = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"])
        assert rel_err(host(Y), ref) <= TOL


@needs_gpu
def test_noalloc_rejects_sizes_over_the_scratch():
    dev()
    T, d, F, n = 2048, 512, 4096, 32
    assert wide.ffn_masked_workspace(T, d, F, n) > wide.binding.NOALLOC_SCRATCH_BYTES
    c = ffn_case("ffn_noalloc_big", T, d, F, n, 0.5, "topk")
    Y = nan_bf16((T, d))
    with pytest.raises(WideError) as e:
        wide.ffn_masked_noalloc(*_args(c), out=Y)
    assert e.value.status == WIDE_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(Y.float()).all(), "a rejected call must launch nothing"
