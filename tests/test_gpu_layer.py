"""GPU parity of wide_layer_masked (pre-norm layer: RMSNorm, masked GQA
attention with RoPE, residual, RMSNorm, masked SwiGLU FFN, residual)."""
import numpy as np
import pytest
import torch

import sparse_wide_mask_amd as wide
from oracle import attn_masked, ffn_masked, layer_masked
from synth import bf16_round
from synth.workloads import layer_case, layer_8b
from tests._gpu import TOL, bf16, dev, host, log, nan_bf16, needs_gpu, rel_err, u8


def gpu_weights(c):
    m = c["meta"]
    return dict(rms1=bf16(c["rms1"]), rms2=bf16(c["rms2"]), Wq=bf16(c["Wq"]), Wk=bf16(c["Wk"]),
                Wv=bf16(c["Wv"]), Wo_packed=wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]),
                W_gate=bf16(c["W_gate"]), W_up=bf16(c["W_up"]),
                W_down_packed=wide.pack_kmajor(bf16(c["W_down"]), m["n_ffn"]))


def gpu_layer(c, W=None, **kw):
    m = c["meta"]
    T, d = c["X"].shape
    Y = nan_bf16((T, d))
    wide.layer_masked(bf16(c["X"]), u8(c["attn_mask"]), u8(c["ffn_mask"]), W or gpu_weights(c),
                      n_q=m["n_q"], n_kv=m["n_kv"], head_dim=128, rope_theta=m["rope_theta"],
                      eps=m["eps"], out=Y, **kw)
    torch.cuda.synchronize()
    return host(Y)


def oracle_layer(c, rows=None, parts=False):
    m = c["meta"]
    return layer_masked(c["X"], c["attn_mask"], c["ffn_mask"], c, n_q=m["n_q"], n_kv=m["n_kv"],
                        head_dim=128, n_ffn=m["n_ffn"], rope_theta=m["rope_theta"], eps=m["eps"],
                        rows=rows, return_parts=parts)


SHAPES = [
    # T, d, F, n_ffn, n_q, n_kv, keep, kind
    (200, 256, 1024, 8, 8, 2, 0.5, "router"),
    (513, 512, 2048, 16, 16, 4, 0.5, "bernoulli"),
    (300, 256, 1536, 12, 8, 8, 0.75, "clustered"),
    (64, 256, 1024, 8, 8, 2, 1.0, "ones"),
    (400, 256, 512, 16, 8, 2, 0.5, "router"),   # FFN groups of 32 channels
    (1, 256, 1024, 8, 8, 2, 0.5, "router"),     # one token
    (17, 320, 640, 10, 8, 2, 0.5, "bernoulli"),  # a few tokens, 192-column K-masked tiles
    # wide rows: the RMSNorm keeps rows of up to 8192 elements in registers between
    # its two passes and reads longer ones again
    (40, 8192, 1024, 8, 8, 2, 0.5, "router"),
    (40, 8256, 1024, 8, 8, 2, 0.5, "bernoulli"),
]


@needs_gpu
@pytest.mark.parametrize("T,d,F,n_ffn,n_q,n_kv,keep,kind", SHAPES)
def test_layer_prefill_shapes(T, d, F, n_ffn, n_q, n_kv, keep, kind):
    dev()
    log(f"layer prefill T={T} d={d} F={F} n_ffn={n_ffn} n_q={n_q} n_kv={n_kv} {kind}")
    c = layer_case(f"layer_{T}_{d}_{kind}", T, d, F, n_ffn, n_q, n_kv, 128, keep, kind)
    got = gpu_layer(c)
    ref, parts = oracle_layer(c, parts=True)
    assert rel_err(got, ref) <= TOL
    # y - x is dominated by the bf16 rounding of y at |x|, so the sublayers are also
    # checked alone, on the oracle's own (bf16-rounded) intermediate inputs
    _check_sublayers(c, parts)


def _check_sublayers(c, parts, rows=None):
    m = c["meta"]
    R = slice(None) if rows is None else rows
    # u = RMSNorm(x) is produced for every token (the attention keys need them all)
    u = bf16_round(parts["u"].astype(np.float32))
    Ya = nan_bf16(u.shape)
    wide.attn_proj_masked(bf16(u), u8(c["attn_mask"]), bf16(c["Wq"]), bf16(c["Wk"]),
                          bf16(c["Wv"]), wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]),
                          n_q=m["n_q"], n_kv=m["n_kv"], rope_theta=m["rope_theta"], out=Ya)
    torch.cuda.synchronize()
    ra = attn_masked(u, c["attn_mask"], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                     n_kv=m["n_kv"], head_dim=128, rope_theta=m["rope_theta"], rows=rows)
    assert rel_err(host(Ya)[R], ra) <= TOL
    w = bf16_round(parts["w"].astype(np.float32))
    fm = c["ffn_mask"][R]
    Yf = nan_bf16(w.shape)
    wide.ffn_masked(bf16(w), u8(fm), bf16(c["W_gate"]), bf16(c["W_up"]),
                    wide.pack_kmajor(bf16(c["W_down"]), m["n_ffn"]), out=Yf)
    torch.cuda.synchronize()
    assert rel_err(host(Yf), ffn_masked(w, fm, c["W_gate"], c["W_up"], c["W_down"])) <= TOL


@needs_gpu
def test_layer_prefill_asymmetric_keep():
    """The pages' asymmetric budget: attention keeps 3 of 8 groups, FFN about 72 % of
    its groups (router masks from the same input)."""
    dev()
    log("layer prefill asymmetric keep")
    c = layer_case("layer_asym", 400, 512, 2048, 16, 16, 8, 128, 0.72, "router", attn_keep=0.34)
    assert c["attn_mask"].sum(axis=1).max() == 3 and c["ffn_mask"].sum(axis=1).max() == 12
    got = gpu_layer(c)
    ref, parts = oracle_layer(c, parts=True)
    assert rel_err(got, ref) <= TOL
    _check_sublayers(c, parts)


@needs_gpu
@pytest.mark.parametrize("kind", ["clustered", "router"])
def test_layer_prefill_8b_ffn_token_sort_bit_identical(kind):
    """The benchmarked layer shape (T = 8192, 112 FFN groups of 128) with the FFN
    token sort (WIDE_FLAG_FFN_TOKEN_SORT): every output element equals the
    unsorted call's bit for bit (the unsorted output is checked against the oracle
    row by row elsewhere); 16 sampled rows against the oracle as well."""
    dev()
    log(f"layer prefill 8B T=8192 {kind} with the FFN token sort")
    c = layer_8b(8192, kind=kind, keep=0.5)
    W = gpu_weights(c)
    plain = gpu_layer(c, W)
    got = gpu_layer(c, W, sort_ffn_tokens=True)
    assert np.array_equal(got.view(np.uint32), plain.view(np.uint32))
    rows = np.sort(np.random.default_rng(9).choice(8192, 16, replace=False))
    ref = oracle_layer(c, rows=rows)
    assert rel_err(got[rows], ref) <= TOL


@needs_gpu
def test_layer_all_zero_masks_is_identity():
    dev()
    c = layer_case("layer_zero", 300, 256, 1024, 8, 8, 2, 128, 0.0, "zeros")
    got = gpu_layer(c)
    assert np.array_equal(got, c["X"]), "all-zero masks must return x bit-exactly"


@needs_gpu
@pytest.mark.parametrize("ffn_group,kind,keep", [(128, "router", 0.5), (64, "router", 0.5),
                                                (128, "clustered", 0.5), (128, "router", 0.25),
                                                (128, "bernoulli", 0.75)])
def test_layer_prefill_llama31_8b_sampled(ffn_group, kind, keep):
    """Full Llama-3.1-8B layer shape at T=8192: router top-k at 50 % with FFN groups of
    128 (112 groups) and of 64 (224 groups, the group-size sweep), router top-k at 25 %
    and Bernoulli at 75 % (the keep sweep), and clustered masks at 50 % (tokens around
    8 prototypes: uneven group counts, which the QKV and attention-core kernels share
    the compute units out by, and few distinct head patterns for the O projection's
    token sort).  The oracle computes 24 sampled token
    rows (keys/values of all tokens).  The attention sublayer (RoPE theta 5e5) and the
    FFN sublayer are also checked alone at this shape on the oracle's intermediate
    inputs (bf16-rounded), where the residual does not hide their error."""
    dev()
    log(f"layer prefill 8B T=8192 G={ffn_group} {kind} keep={keep} (sampled)")
    c = layer_8b(8192, ffn_group=ffn_group, kind=kind, keep=keep)
    m = c["meta"]
    rows = np.sort(np.random.default_rng(2).choice(8192, 24, replace=False))
    rows[0], rows[-1] = 0, 8191
    got = gpu_layer(c)
    assert np.all(np.isfinite(got))
    ref, parts = oracle_layer(c, rows=rows, parts=True)
    assert rel_err(got[rows], ref) <= TOL
    # attention on u = RMSNorm(x), FFN on w = RMSNorm(h) of the oracle (sampled rows)
    _check_sublayers(c, parts, rows=rows)


# Per-row bound of the every-row check.  The parity bar is TOL on max|err| / max|ref|
# over the whole output; row by row the bf16 operands of the attention (P and V in
# the P V product, O into the output projection) leave rows with small outputs up to
# about 1 % off (measured worst of 8192 rows: 1.0e-2 attention, 4.6e-3 FFN), while a
# row computed from the wrong tokens or groups is off by its own magnitude.
ROW_TOL = 2.5e-2


def _rowwise(got, ref, tol):
    """Per token row: max|err| / max|ref| <= tol; a row the oracle gives as exact zeros
    (every group dropped) must be exact zeros."""
    scale = np.abs(ref).max(axis=1)
    err = np.abs(got - ref).max(axis=1)
    zero = scale == 0
    assert np.all(got[zero] == 0), "a row with every group dropped is not exactly zero"
    worst = (err[~zero] / scale[~zero]).max(initial=0.0)
    assert worst <= tol, f"worst row {worst:.3e}"
    return worst


@needs_gpu
def test_layer_prefill_llama31_8b_every_row():
    """The benchmarked shape (Llama-3.1-8B layer, T = 8192, router masks keeping 50 %)
    on EVERY token row, against the oracle run in float32 (the same code as the fp64
    oracle; fp32 changes its results by about 1e-6 relative, four orders below the
    tolerance, and runs the whole layer in seconds).  Checked per row: the layer
    output y, and the attention and FFN sublayers alone on the oracle's intermediate
    inputs, where the residual does not hide their error."""
    dev()
    log("layer prefill 8B T=8192, every row against the fp32 oracle")
    c = layer_8b(8192)
    m = c["meta"]
    got = gpu_layer(c)
    assert np.all(np.isfinite(got))
    ref, parts = layer_masked(c["X"], c["attn_mask"], c["ffn_mask"], c, n_q=m["n_q"],
                              n_kv=m["n_kv"], head_dim=128, n_ffn=m["n_ffn"],
                              rope_theta=m["rope_theta"], eps=m["eps"], dtype=np.float32,
                              return_parts=True)
    assert rel_err(got, ref) <= TOL
    _rowwise(got, ref, ROW_TOL)
    # attention sublayer alone on u, every row
    u = bf16_round(parts["u"].astype(np.float32))
    Ya = nan_bf16(u.shape)
    wide.attn_proj_masked(bf16(u), u8(c["attn_mask"]), bf16(c["Wq"]), bf16(c["Wk"]),
                          bf16(c["Wv"]), wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]),
                          n_q=m["n_q"], n_kv=m["n_kv"], rope_theta=m["rope_theta"], out=Ya)
    torch.cuda.synchronize()
    ra = attn_masked(u, c["attn_mask"], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                     n_kv=m["n_kv"], head_dim=128, rope_theta=m["rope_theta"], dtype=np.float32)
    assert rel_err(host(Ya), ra) <= TOL
    log(f"  attention sublayer, worst row {_rowwise(host(Ya), ra, ROW_TOL):.2e}")
    # FFN sublayer alone on w, every row
    w = bf16_round(parts["w"].astype(np.float32))
    Yf = nan_bf16(w.shape)
    wide.ffn_masked(bf16(w), u8(c["ffn_mask"]), bf16(c["W_gate"]), bf16(c["W_up"]),
                    wide.pack_kmajor(bf16(c["W_down"]), m["n_ffn"]), out=Yf)
    torch.cuda.synchronize()
    rf = ffn_masked(w, c["ffn_mask"], c["W_gate"], c["W_up"], c["W_down"], dtype=np.float32)
    assert rel_err(host(Yf), rf) <= TOL
    log(f"  FFN sublayer, worst row {_rowwise(host(Yf), rf, ROW_TOL):.2e}")


@needs_gpu
def test_layer_prefill_back_to_back_shared_workspace():
    """Two layer calls enqueued back to back on one stream with one workspace, with
    different inputs and masks: the second call's reorders overwrite buffers that the
    first call's kernels read, and stream order keeps them apart.  Both outputs match
    the oracle."""
    dev()
    log("layer prefill, two calls back to back on one workspace")
    T, d, F, n_ffn, n_q, n_kv = 1024, 512, 2048, 16, 16, 4
    cases = [layer_case(f"layer_b2b_{kind}", T, d, F, n_ffn, n_q, n_kv, 128, 0.5, kind)
             for kind in ("router", "bernoulli")]
    ws = torch.empty(wide.layer_masked_workspace(T, d, F, n_ffn, n_q, n_kv), dtype=torch.uint8,
                     device=dev())
    # every input on the device first, so that nothing between the calls waits
    args = [(bf16(c["X"]), u8(c["attn_mask"]), u8(c["ffn_mask"]), gpu_weights(c), nan_bf16((T, d)))
            for c in cases]
    torch.cuda.synchronize()
    for c, (X, am, fm, W, Y) in zip(cases, args):
        m = c["meta"]
        wide.layer_masked(X, am, fm, W, n_q=n_q, n_kv=n_kv, head_dim=128,
                          rope_theta=m["rope_theta"], eps=m["eps"], out=Y, workspace=ws)
    outs = [a[-1] for a in args]
    torch.cuda.synchronize()
    for c, Y in zip(cases, outs):
        assert rel_err(host(Y), oracle_layer(c)) <= TOL


@needs_gpu
def test_layer_prefill_max_tokens_sampled():
    """The whole layer at the maximum token count, 65536, at a small width (d = 256,
    d_ff = 1024 in 8 groups, 8 query and 8 KV heads, router masks keeping 50 %):
    48 sampled rows against the oracle; every row finite."""
    dev()
    T = 65536
    log(f"layer prefill T={T} (maximum), sampled")
    c = layer_case("layer_max", T, 256, 1024, 8, 8, 8, 128, 0.5, "router")
    got = gpu_layer(c)
    assert np.all(np.isfinite(got))
    rows = np.sort(np.random.default_rng(5).choice(T, 48, replace=False))
    rows[0], rows[-1] = 0, T - 1
    assert rel_err(got[rows], oracle_layer(c, rows=rows)) <= TOL
