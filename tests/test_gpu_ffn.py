"""GPU parity of wide_ffn_masked (prefill) against the oracle.

Outputs are NaN-filled before the call so an unwritten element fails; the bar
is max|err| / max|ref| <= 1e-2 per output (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import ffn_masked
from synth.workloads import ffn_case, ffn_prefill_3b, tiny_ffn
from tests._gpu import TOL, bf16, dev, host, log, nan_bf16, needs_gpu, rel_err, u8


def _gpu_ffn(c, mode="prefill", sort_tokens=False):
    n = c["mask"].shape[1]
    T, d = c["X"].shape
    Y = nan_bf16((T, d))
    wide.ffn_masked(bf16(c["X"]), u8(c["mask"]), bf16(c["W_gate"]), bf16(c["W_up"]),
                    wide.pack_kmajor(bf16(c["W_down"]), n), mode=mode, out=Y,
                    sort_tokens=sort_tokens)
    torch.cuda.synchronize()
    return host(Y)


@needs_gpu
@pytest.mark.parametrize("n,G,d", [(5, 128, 192), (7, 32, 192), (3, 64, 64)])
def test_pack_kmajor_is_the_blockwise_transpose(n, G, d):
    dev()
    r = np.random.default_rng(0)
    from synth import bf16_round
    W = bf16_round(r.standard_normal((n * G, d)).astype(np.float32))
    P = host(wide.pack_kmajor(bf16(W), n))
    assert np.array_equal(P, W.reshape(n, G, d).transpose(0, 2, 1))


@needs_gpu
def test_tiny_fp32_configuration_raw_input_difference():
    """The tiny configuration is declared fp32; the library computes on its inputs
    rounded to bf16.  Parity is judged on the rounded inputs (the oracle in fp64, and
    in fp32); the difference to the oracle on the raw fp32 inputs is reported and must
    stay within the bf16 input rounding's own effect (the fp64 oracle on rounded
    against raw inputs) plus the tolerance."""
    dev()
    from synth import normal
    c = tiny_ffn()
    raw = {k: normal("tiny_ffn", k, c[k].shape, 1.0 if k == "X" else 0.02, round_bf16=False)
           for k in ("X", "W_gate", "W_up", "W_down")}
    assert all(np.array_equal(np.asarray(raw[k], np.float32), np.asarray(raw[k])) for k in raw)
    got = _gpu_ffn(c)
    ref64 = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"])
    ref32 = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"], dtype=np.float32)
    raw64 = ffn_masked(raw["X"], c["mask"], raw["W_gate"], raw["W_up"], raw["W_down"])
    e64, e32, eraw = rel_err(got, ref64), rel_err(got, ref32), rel_err(got, raw64)
    e_round = rel_err(ref64, raw64)
    log(f"tiny fp32 configuration: GPU vs oracle fp64 {e64:.2e}, vs oracle fp32 {e32:.2e}, "
        f"vs oracle on raw fp32 inputs {eraw:.2e}; oracle rounded vs raw inputs {e_round:.2e}; "
        f"oracle fp32 vs fp64 {rel_err(ref32, ref64):.2e}")
    assert e64 <= TOL and e32 <= TOL
    assert eraw <= e_round + TOL


@needs_gpu
def test_tiny_ffn():
    dev()
    c = tiny_ffn()
    log("tiny ffn T=64 d=256 F=1024 n=16")
    got = _gpu_ffn(c)
    ref = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"])
    assert rel_err(got, ref) <= TOL


SHAPES = [
    # T, d, F, n, keep, kind   (several tiles and ragged tails in T, 64- and 128-wide groups)
    (300, 256, 1024, 8, 0.5, "topk"),
    (513, 512, 2048, 16, 0.5, "bernoulli"),
    (777, 384, 1536, 12, 0.25, "clustered"),
    (1024, 256, 2048, 32, 0.75, "topk"),
    (130, 320, 640, 10, 0.5, "bernoulli"),
    (257, 256, 1024, 8, 1.0, "ones"),
    (257, 256, 1024, 8, 0.0, "zeros"),
    (1, 256, 1024, 16, 0.5, "topk"),
    # groups of 32 channels: 64-wide FFN up tiles; FFN down K slices over pairs of groups
    (300, 256, 512, 16, 0.5, "topk"),
    (1100, 512, 1024, 32, 0.75, "bernoulli"),
    (257, 256, 2048, 64, 0.25, "clustered"),
    (129, 384, 256, 8, 1.0, "ones"),
    # uneven group counts over a multiple of 8 groups
    (2000, 256, 2048, 16, 0.5, "clustered"),
    # groups of 256 channels: two FFN up channel tiles per group, each with its own tails
    (600, 256, 2048, 8, 0.5, "bernoulli"),
]


@needs_gpu
@pytest.mark.parametrize("T,d,F,n,keep,kind", SHAPES)
def test_ffn_prefill_shapes(T, d, F, n, keep, kind):
    dev()
    log(f"ffn prefill T={T} d={d} F={F} n={n} keep={keep} {kind}")
    c = ffn_case(f"ffn_{T}_{d}_{F}_{n}_{kind}", T, d, F, n, keep, kind)
    got = _gpu_ffn(c)
    ref = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"])
    if kind == "zeros":
        assert np.all(got == 0.0)
    assert rel_err(got, ref) <= TOL


@needs_gpu
@pytest.mark.parametrize("T,d,F,n,keep,kind", [
    (777, 384, 1536, 12, 0.25, "clustered"),   # 12 groups: key of the first 8
    (2000, 256, 2048, 16, 0.5, "clustered"),
    (257, 256, 2048, 64, 0.25, "clustered"),   # groups of 32: pairs per K slice
    (1100, 512, 1024, 32, 0.75, "bernoulli"),
    (600, 256, 2048, 8, 0.5, "bernoulli"),     # 8 groups: the whole pattern
    (1, 256, 1024, 16, 0.5, "topk"),
])
def test_ffn_token_sort_bit_identical(T, d, F, n, keep, kind):
    """WIDE_FLAG_FFN_TOKEN_SORT: the down projection over tokens sorted by their
    first groups' pattern, each tile over the union of its own rows.  A token's
    sum runs over its kept groups in ascending order in any tile, so the output
    equals the unsorted call's bit for bit; and the oracle's within tolerance."""
    dev()
    log(f"ffn token sort T={T} d={d} F={F} n={n} keep={keep} {kind}")
    c = ffn_case(f"ffn_sort_{T}_{d}_{F}_{n}_{kind}", T, d, F, n, keep, kind)
    plain = _gpu_ffn(c)
    got = _gpu_ffn(c, sort_tokens=True)
    assert np.array_equal(got.view(np.uint32), plain.view(np.uint32))
    ref = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"])
    assert rel_err(got, ref) <= TOL


@needs_gpu
def test_ffn_up_last_tile_sizes():
    """Per-group kept counts placed at the boundaries of the up projection's row
    tiles (256 rows) and of its tail parts (64-row tiles for a last tile of at most
    128 rows): 0, 1, 64, 65, 128, 129, 356 and 639 kept tokens in the 8 groups of
    128 channels, so last tiles of 1, 64, 65, 128, 129, 100 and 127 rows."""
    dev()
    T, d, F, n = 700, 256, 1024, 8
    counts = [0, 1, 64, 65, 128, 129, 356, 639]
    log(f"ffn prefill T={T} per-group counts {counts}")
    c = ffn_case("ffn_tail_sizes", T, d, F, n, 0.5, "bernoulli")
    r = np.random.default_rng(11)
    mask = np.zeros((T, n), np.uint8)
    for g, k in enumerate(counts):
        mask[r.choice(T, k, replace=False), g] = 1
    c["mask"] = mask
    got = _gpu_ffn(c)
    ref = ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"])
    assert rel_err(got, ref) <= TOL
    assert np.array_equal(got[mask.sum(1) == 0], np.zeros((int((mask.sum(1) == 0).sum()), d)))


@needs_gpu
def test_ffn_prefill_llama32_3b_sampled():
    """Full Llama-3.2-3B FFN prefill shape (T=4096, d=3072, d_ff=8192, 64 groups,
    router top-k 32 of 64); the oracle computes 96 sampled token rows (rows are
    independent) and every output row is checked finite."""
    dev()
    log("ffn prefill 3B full size")
    c = ffn_prefill_3b()
    got = _gpu_ffn(c)
    assert np.all(np.isfinite(got))
    rows = np.sort(np.random.default_rng(1).choice(4096, 96, replace=False))
    rows[0], rows[-1] = 0, 4095
    ref = ffn_masked(c["X"][rows], c["mask"][rows], c["W_gate"], c["W_up"], c["W_down"])
    assert rel_err(got[rows], ref) <= TOL


@needs_gpu
def test_ffn_prefill_max_tokens_sampled():
    """The maximum token count, 65536, at a small width (d = 256, d_ff = 1024 in 8
    groups of 128, top-k 4 of 8): about 128 row tiles per group and group tails at
    the end of the grid in the up projection, 256 row tiles in the down
    projection.  64 sampled rows against the oracle; every row finite."""
    dev()
    T = 65536
    log(f"ffn prefill T={T} (maximum), sampled")
    c = ffn_case("ffn_max", T, 256, 1024, 8, 0.5, "topk")
    got = _gpu_ffn(c)
    assert np.all(np.isfinite(got))
    rows = np.sort(np.random.default_rng(4).choice(T, 64, replace=False))
    rows[0], rows[-1] = 0, T - 1
    ref = ffn_masked(c["X"][rows], c["mask"][rows], c["W_gate"], c["W_up"], c["W_down"])
    assert rel_err(got[rows], ref) <= TOL


@needs_gpu
def test_ffn_prefill_3b_groups_of_32_sampled():
    """The Llama-3.2-3B FFN shape (T=4096, d=3072, d_ff=8192) in 256 groups of 32
    channels, the most groups the library takes, router-style top-k 128 of 256:
    64 sampled rows against the oracle; every row finite."""
    dev()
    log("ffn prefill 3B, 256 groups of 32 (sampled)")
    c = ffn_case("ffn_3b_g32", 4096, 3072, 8192, 256, 0.5, "topk")
    got = _gpu_ffn(c)
    assert np.all(np.isfinite(got))
    rows = np.sort(np.random.default_rng(6).choice(4096, 64, replace=False))
    rows[0], rows[-1] = 0, 4095
    ref = ffn_masked(c["X"][rows], c["mask"][rows], c["W_gate"], c["W_up"], c["W_down"])
    assert rel_err(got[rows], ref) <= TOL
