#!/usr/bin/env python3
"""Benchmark of WIDE masked dynamic-width execution on one MI355X.

A step is one pass of the whole masked path over one batch of synthetic input.
The default workload is one Llama-3.1-8B-shaped decoder layer in prefill
(T = 8192 tokens, d_model 4096, 32 query / 8 KV heads of 128, d_ff 14336 in 112
FFN groups of 128, RoPE theta 5e5), whose masks keep 50% of the attention groups
and 50% of the FFN groups per token (router top-k on the layer input).  The step
runs mask reordering, RMSNorm, the masked QKV projections, the causal attention
core, the masked output projection, RMSNorm, the masked SwiGLU up and down
projections, and both residual adds.

Output: one JSON line (metric, value = masked tokens/s and ms per step over K
uninstrumented steps, the roofline of the dominant kernel timed by HIP events on
the library's streams over K more steps with a trace on, the same kernels with
all-ones masks, per-kernel times, and the CPU oracle timed on a bounded sample of
the same inputs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "masked tokens/s + % of MFMA (prefill) / HBM (decode) roofline at 50% sparsity"
HD = 128
ORACLE_DTYPE = np.float32   # the CPU baseline times the oracle in fp32 (its parity runs use fp64)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------- workloads

def layer_name(base, keep, kind, ffn_group=128, attn_keep=None):
    """Workload name; the default structure (router top-k at 50%, FFN groups of 128) keeps
    the base name."""
    name = base if (kind, keep) == ("router", 0.5) else f"{base}_{kind}_{int(round(keep * 100))}"
    if attn_keep is not None:
        name += f"_attn{int(round(attn_keep * 100))}"
    return name if ffn_group == 128 else f"{name}_g{ffn_group}"


def measured_keep(c):
    """Kept fraction of (token, group) pairs and the batch union, per mask."""
    out = {}
    for k in ("attn_mask", "ffn_mask"):
        m = c[k] != 0
        out[f"{k}_keep"] = round(float(m.mean()), 4)
        out[f"{k}_union"] = int(m.any(axis=0).sum())
    return out


class LayerPrefill:
    """Llama-3.1-8B-shaped decoder layer, prefill."""

    sort_ffn = False  # WIDE_FLAG_FFN_TOKEN_SORT (bench.py --sort-ffn)

    def __init__(self, T=8192, keep=0.5, kind="router", ffn_group=128, attn_keep=None):
        from synth.workloads import layer_8b
        self.name = layer_name("layer_prefill_8b", keep, kind, ffn_group, attn_keep)
        self.c = layer_8b(T, keep=keep, kind=kind, ffn_group=ffn_group, attn_keep=attn_keep)
        m = self.c["meta"]
        self.m = m
        self.T = T
        self.config = dict(workload=self.name, T=T, d_model=m["d"], d_ff=m["F"],
                           n_ffn_groups=m["n_ffn"], n_q_heads=m["n_q"], n_kv_heads=m["n_kv"],
                           head_dim=HD, rope_theta=m["rope_theta"], keep=keep,
                           masks=f"{kind} top-k" if kind == "router" else kind,
                           **measured_keep(self.c))

    def upload(self, torch, wide, bf16, u8):
        c, m = self.c, self.m
        self.W = dict(rms1=bf16(c["rms1"]), rms2=bf16(c["rms2"]), Wq=bf16(c["Wq"]), Wk=bf16(c["Wk"]),
                      Wv=bf16(c["Wv"]), Wo_packed=wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]),
                      W_gate=bf16(c["W_gate"]), W_up=bf16(c["W_up"]),
                      W_down_packed=wide.pack_kmajor(bf16(c["W_down"]), m["n_ffn"]))
        self.X = bf16(c["X"])
        self.masks = (u8(c["attn_mask"]), u8(c["ffn_mask"]))
        self.ones = (torch.ones_like(self.masks[0]), torch.ones_like(self.masks[1]))
        self.Y = torch.empty_like(self.X)
        ws = wide.layer_masked_workspace(self.T, m["d"], m["F"], m["n_ffn"], m["n_q"], m["n_kv"],
                                         HD, m["rope_theta"], m["eps"])
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.wide = wide

    def step(self, ones=False):
        m = self.m
        am, fm = self.ones if ones else self.masks
        self.wide.layer_masked(self.X, am, fm, self.W, n_q=m["n_q"], n_kv=m["n_kv"], head_dim=HD,
                               rope_theta=m["rope_theta"], eps=m["eps"], out=self.Y,
                               workspace=self.ws, sort_ffn_tokens=self.sort_ffn)

    def work(self, ones=False):
        """Algorithmic FLOPs per launch of each kernel, from the actual masks."""
        m = self.m
        d, F, n_ffn, n_q, n_kv = m["d"], m["F"], m["n_ffn"], m["n_q"], m["n_kv"]
        G, r = F // n_ffn, n_q // n_kv
        am = np.ones_like(self.c["attn_mask"]) if ones else self.c["attn_mask"]
        fm = np.ones_like(self.c["ffn_mask"]) if ones else self.c["ffn_mask"]
        kf = float((fm != 0).sum())
        cnt = (am != 0).sum(axis=0).astype(np.float64)
        ka = float(cnt.sum())
        pairs = float((cnt * (cnt + 1) / 2).sum())       # causal (query, key) pairs per group
        return {
            "ffn_up_prefill": 2 * 2 * d * G * kf,          # gate and up
            "ffn_down": 2 * d * G * kf,
            "attn_qkv_prefill": 2 * d * (r + 2) * HD * ka,
            "attn_core_prefill": 4 * HD * r * pairs,       # QK^T and PV
            "attn_o": 2 * d * r * HD * ka,
        }

    def oracle_sample(self, S):
        """The dense oracle on the first S tokens of the same inputs (causal: these
        rows of the layer output depend on nothing later)."""
        from oracle import layer_masked
        c, m = self.c, self.m
        W = {k: c[k] for k in ("rms1", "rms2", "Wq", "Wk", "Wv", "Wo", "W_gate", "W_up", "W_down")}
        t0 = time.perf_counter()
        layer_masked(c["X"][:S], c["attn_mask"][:S], c["ffn_mask"][:S], W, n_q=m["n_q"],
                     n_kv=m["n_kv"], head_dim=HD, n_ffn=m["n_ffn"], rope_theta=m["rope_theta"],
                     eps=m["eps"], dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


class LayerPrefillRouted(LayerPrefill):
    """LayerPrefill with the masks chosen on the GPU inside the step: the layer input's
    two linear routers (R_attn [8, d], R_ffn [112, d], the input generator's router
    weights rounded to bf16) keep 4 of 8 head groups and 56 of 112 FFN groups, and
    their packed words go straight to the mask reorders (wide_layer_masked_routed)."""

    def __init__(self, T=8192, keep=0.5, kind="router", ffn_group=128, attn_keep=None):
        super().__init__(T, keep, "router", ffn_group, attn_keep)
        from synth import bf16_round, normal
        m, c = self.m, self.c
        cfg = f"layer_8b_pre_router_{int(round(keep * 100))}"
        # the generator's routers: logits x @ R with R [d, n]; the GPU takes R^T [n, d]
        self.R_attn = bf16_round(normal(cfg, "attn_mask.R", (m["d"], m["n_kv"]), 1.0 / 64,
                                        round_bf16=False).T)
        self.R_ffn = bf16_round(normal(cfg, "ffn_mask.R", (m["d"], m["n_ffn"]), 1.0 / 64,
                                       round_bf16=False).T)
        self.k_attn = int(round((attn_keep if attn_keep is not None else keep) * m["n_kv"]))
        self.k_ffn = int(round(keep * m["n_ffn"]))
        self.name = self.name.replace("layer_prefill_8b", "layer_prefill_8b_routed", 1)
        self.config.update(workload=self.name, masks="GPU router top-k (in the step)")

    def upload(self, torch, wide, bf16, u8):
        super().upload(torch, wide, bf16, u8)
        m = self.m
        self.Ra, self.Rf = wide.pack_router(bf16(self.R_attn)), wide.pack_router(bf16(self.R_ffn))
        # mask outputs: one pair for the masked steps, one for the all-ones steps
        self.masks_out = [(torch.empty((self.T, m["n_kv"]), dtype=torch.uint8, device="cuda"),
                           torch.empty((self.T, m["n_ffn"]), dtype=torch.uint8, device="cuda"))
                          for _ in range(2)]
        self.am, self.fm = self.masks_out[0]

    def step(self, ones=False):
        m = self.m
        ka, kf = (m["n_kv"], m["n_ffn"]) if ones else (self.k_attn, self.k_ffn)
        am, fm = self.masks_out[1 if ones else 0]
        self.wide.layer_masked_routed(self.X, self.Ra, ka, self.Rf, kf, self.W, n_q=m["n_q"],
                                      n_kv=m["n_kv"], n_ffn=m["n_ffn"], head_dim=HD,
                                      rope_theta=m["rope_theta"], eps=m["eps"], out=self.Y,
                                      attn_mask=am, ffn_mask=fm, workspace=self.ws,
                                      sort_ffn_tokens=self.sort_ffn)

    def work(self, ones=False):
        # counted from the masks the GPU routers chose (read back after the run)
        if not ones and self.am is not None:
            self.c = dict(self.c, attn_mask=self.am.cpu().numpy(), ffn_mask=self.fm.cpu().numpy())
            self.config.update(measured_keep(self.c))
        return super().work(ones)


class LayerDecodeMaskedCache:
    """Llama-3.1-8B-shaped layer decode over masked caches: batch 32 at position 8192,
    each (sequence, group) cache holding only the earlier tokens that kept the group
    (binomial(8192, 1/2) entries at keep 4 of 8); wide_layer_decode_masked_cache.
    All-ones comparison: every group kept, every cache full."""

    def __init__(self, B=32, pos=8192, keep=0.5, kind="router", ffn_group=128, attn_keep=None):
        self.inner = LayerDecode(B, pos, keep, kind, ffn_group, attn_keep)
        self.c, self.m, self.T, self.pos = self.inner.c, self.inner.m, B, pos
        rng = np.random.default_rng(8193)
        self.lens = rng.binomial(pos, 0.5, size=(B, self.m["n_kv"])).astype(np.int32)
        self.name = self.inner.name.replace("layer_decode_8b", "layer_decode_masked_cache_8b", 1)
        self.config = dict(self.inner.config, workload=self.name, position=pos,
                           kv_cap=pos + 1, mean_cache_len=round(float(self.lens.mean()), 1))
        self.config.pop("kv_len", None)
        self.bound = "hbm"

    def upload(self, torch, wide, bf16, u8):
        self.inner.upload(torch, wide, bf16, u8)
        self.L = torch.from_numpy(self.lens).cuda()
        self.full = torch.full_like(self.L, self.pos)
        self.wide = wide

    def step(self, ones=False):
        inn, m = self.inner, self.m
        S = inn.sets[inn.i % len(inn.sets)]
        inn.i += 1
        am, fm = inn.ones if ones else inn.masks
        self.wide.layer_decode_masked_cache(inn.X, am, fm, S, n_q=m["n_q"], n_kv=m["n_kv"],
                                            K_cache=S["K_cache"], V_cache=S["V_cache"],
                                            kv_len=self.full if ones else self.L, pos=self.pos,
                                            head_dim=HD, rope_theta=m["rope_theta"],
                                            eps=m["eps"], out=inn.Y, workspace=inn.ws)

    def work(self, ones=False):
        w = self.inner.work(ones)
        m = self.m
        am = np.ones_like(self.c["attn_mask"]) if ones else (self.c["attn_mask"] != 0)
        lens = np.full_like(self.lens, self.pos) if ones else self.lens
        r = m["n_q"] // m["n_kv"]
        w["attn_core_decode"] = (float(((lens + 1) * am).sum()) * 2 * HD * 2
                                 + float(am.sum()) * r * HD * 2)
        return w

    def oracle_sample(self, S):
        from oracle import layer_masked
        c, m = self.c, self.m
        W = {k: c[k] for k in ("rms1", "rms2", "Wq", "Wk", "Wv", "Wo", "W_gate", "W_up", "W_down")}
        t0 = time.perf_counter()
        layer_masked(c["X"][:S], c["attn_mask"][:S], c["ffn_mask"][:S], W, n_q=m["n_q"],
                     n_kv=m["n_kv"], head_dim=HD, n_ffn=m["n_ffn"], rope_theta=m["rope_theta"],
                     eps=m["eps"], decode=True, K_cache=c["K_cache"][:S], V_cache=c["V_cache"][:S],
                     kv_len=self.lens[:S], pos=self.pos, dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


class FfnPrefill:
    """Llama-3.2-3B-shaped FFN prefill (T=4096, d=3072, d_ff=8192 in 64 groups of 128,
    or groups of ffn_group channels)."""

    def __init__(self, T=4096, ffn_group=128):
        from synth.workloads import ffn_prefill_3b
        self.name = "ffn_prefill_3b" + ("" if ffn_group == 128 else f"_g{ffn_group}")
        self.c = ffn_prefill_3b(T, ffn_group)
        m = self.c["meta"]
        self.m, self.T = m, T
        self.config = dict(workload=self.name, T=T, d_model=m["d"], d_ff=m["F"], n_groups=m["n"],
                           keep=m["keep"], masks="router top-k")

    def upload(self, torch, wide, bf16, u8):
        c, m = self.c, self.m
        self.X, self.Wg, self.Wu = bf16(c["X"]), bf16(c["W_gate"]), bf16(c["W_up"])
        self.Wd = wide.pack_kmajor(bf16(c["W_down"]), m["n"])
        self.mask = u8(c["mask"])
        self.ones = torch.ones_like(self.mask)
        self.Y = torch.empty_like(self.X)
        self.ws = torch.empty(wide.ffn_masked_workspace(self.T, m["d"], m["F"], m["n"]),
                              dtype=torch.uint8, device="cuda")
        self.wide = wide

    def step(self, ones=False):
        self.wide.ffn_masked(self.X, self.ones if ones else self.mask, self.Wg, self.Wu, self.Wd,
                             out=self.Y, workspace=self.ws)

    def work(self, ones=False):
        m = self.m
        G = m["F"] // m["n"]
        k = float(self.T * m["n"]) if ones else float((self.c["mask"] != 0).sum())
        return {"ffn_up_prefill": 4 * m["d"] * G * k, "ffn_down": 2 * m["d"] * G * k}

    def oracle_sample(self, S):
        from oracle import ffn_masked
        c = self.c
        t0 = time.perf_counter()
        ffn_masked(c["X"][:S], c["mask"][:S], c["W_gate"], c["W_up"], c["W_down"],
                   dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


class AttnPrefill:
    """Llama-3.1-8B-shaped attention sublayer, prefill T=2048, no RoPE."""

    def __init__(self, T=2048):
        from synth.workloads import attn_prefill_8b
        self.name = "attn_prefill_8b"
        self.c = attn_prefill_8b(T)
        m = self.c["meta"]
        self.m, self.T = m, T
        self.config = dict(workload=self.name, T=T, d_model=m["d"], n_q_heads=m["n_q"],
                           n_kv_heads=m["n_kv"], head_dim=HD, keep=m["keep"], masks="top-k")

    def upload(self, torch, wide, bf16, u8):
        c, m = self.c, self.m
        self.X = bf16(c["X"])
        self.Wq, self.Wk, self.Wv = bf16(c["Wq"]), bf16(c["Wk"]), bf16(c["Wv"])
        self.Wo = wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"])
        self.mask = u8(c["mask"])
        self.ones = torch.ones_like(self.mask)
        self.Y = torch.empty_like(self.X)
        self.ws = torch.empty(wide.attn_proj_masked_workspace(self.T, m["d"], m["n_q"], m["n_kv"]),
                              dtype=torch.uint8, device="cuda")
        self.wide = wide

    def step(self, ones=False):
        m = self.m
        self.wide.attn_proj_masked(self.X, self.ones if ones else self.mask, self.Wq, self.Wk,
                                   self.Wv, self.Wo, n_q=m["n_q"], n_kv=m["n_kv"], out=self.Y,
                                   workspace=self.ws)

    def work(self, ones=False):
        m = self.m
        r = m["n_q"] // m["n_kv"]
        am = np.ones_like(self.c["mask"]) if ones else self.c["mask"]
        cnt = (am != 0).sum(axis=0).astype(np.float64)
        ka, pairs = float(cnt.sum()), float((cnt * (cnt + 1) / 2).sum())
        return {"attn_qkv_prefill": 2 * m["d"] * (r + 2) * HD * ka,
                "attn_core_prefill": 4 * HD * r * pairs, "attn_o": 2 * m["d"] * r * HD * ka}

    def oracle_sample(self, S):
        from oracle import attn_masked
        c, m = self.c, self.m
        t0 = time.perf_counter()
        attn_masked(c["X"][:S], c["mask"][:S], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                    n_kv=m["n_kv"], head_dim=HD, dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


# ---------------------------------------------------------------- decode
#
# Decode is bound by HBM: its work is counted in bytes actually touched (the weight
# blocks of the groups some token of the batch keeps, the K/V of the kept
# (token, group) pairs, activations).  Several copies of the inputs rotate between
# steps so the 256 MB Infinity Cache cannot serve a repeated step.

MALL_BYTES = 256 << 20


def _copies(set_bytes):
    return max(2, -(-(4 * MALL_BYTES) // max(set_bytes, 1)))


class FfnDecode:
    """Llama-3.1-8B-shaped FFN decode: B single tokens, d=4096, d_ff=14336 in 112 groups."""

    def __init__(self, B=1):
        from synth.workloads import ffn_decode_8b
        self.name = f"ffn_decode_8b_B{B}"
        self.c = ffn_decode_8b(B)
        m = self.c["meta"]
        self.m, self.T = m, B
        self.config = dict(workload=self.name, B=B, d_model=m["d"], d_ff=m["F"], n_groups=m["n"],
                           keep=m["keep"], masks="top-k")
        self.bound = "hbm"

    def upload(self, torch, wide, bf16, u8):
        c, m = self.c, self.m
        set_bytes = 3 * m["F"] * m["d"] * 2
        self.sets = []
        for _ in range(_copies(set_bytes)):
            self.sets.append((bf16(c["W_gate"]), bf16(c["W_up"]),
                              wide.pack_kmajor(bf16(c["W_down"]), m["n"])))
        self.X = bf16(c["X"])
        self.mask = u8(c["mask"])
        self.ones = torch.ones_like(self.mask)
        self.Y = torch.empty_like(self.X)
        self.ws = torch.empty(wide.ffn_masked_workspace(self.T, m["d"], m["F"], m["n"], "decode"),
                              dtype=torch.uint8, device="cuda")
        self.wide, self.i = wide, 0

    def step(self, ones=False):
        Wg, Wu, Wd = self.sets[self.i % len(self.sets)]
        self.i += 1
        self.wide.ffn_masked(self.X, self.ones if ones else self.mask, Wg, Wu, Wd, mode="decode",
                             out=self.Y, workspace=self.ws)

    def work(self, ones=False):
        m = self.m
        d, G, B = m["d"], m["F"] // m["n"], self.T
        mk = np.ones_like(self.c["mask"]) if ones else (self.c["mask"] != 0)
        U = float(mk.any(axis=0).sum())
        kept = float(mk.sum())
        return {"ffn_up_decode": U * 2 * G * d * 2 + B * d * 2 + kept * G * 2,
                "ffn_down_decode": U * G * d * 2 + kept * G * 2 + B * d * 2}

    def oracle_sample(self, S):
        from oracle import ffn_masked
        c = self.c
        t0 = time.perf_counter()
        ffn_masked(c["X"][:S], c["mask"][:S], c["W_gate"], c["W_up"], c["W_down"],
                   dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


def _attn_decode_bytes(m, am, d, L):
    """Touched bytes of the attention decode kernels (keys 0..L incl. the new one)."""
    n_q, n_kv = m["n_q"], m["n_kv"]
    r = n_q // n_kv
    B = am.shape[0]
    U = float(am.any(axis=0).sum())
    kept = float(am.sum())
    return {
        "attn_qkv_decode": U * (r + 2) * HD * d * 2 + B * d * 2 + kept * (r + 2) * HD * 2,
        "attn_core_decode": kept * 2 * (L + 1) * HD * 2 + kept * r * HD * 2,
        "attn_o_decode": U * r * HD * d * 2 + kept * r * HD * 2 + B * d * 2,
    }


class AttnDecode:
    """Llama-3.1-8B-shaped attention decode: batch 16 over a 4096-entry cache."""

    def __init__(self, B=16, L=4096):
        from synth.workloads import attn_decode_8b
        self.name = "attn_decode_8b"
        self.c = attn_decode_8b(B, L)
        m = self.c["meta"]
        self.m, self.T, self.L = m, B, L
        self.config = dict(workload=self.name, B=B, kv_len=L, d_model=m["d"], n_q_heads=m["n_q"],
                           n_kv_heads=m["n_kv"], head_dim=HD, keep=m["keep"], masks="top-k")
        self.bound = "hbm"

    def upload(self, torch, wide, bf16, u8):
        c, m = self.c, self.m
        set_bytes = (2 * m["n_q"] + 2 * m["n_kv"]) * HD * m["d"] * 2 + 2 * c["K_cache"].size * 2
        self.sets = []
        for _ in range(_copies(set_bytes)):
            self.sets.append((bf16(c["Wq"]), bf16(c["Wk"]), bf16(c["Wv"]),
                              wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]), bf16(c["K_cache"]),
                              bf16(c["V_cache"])))
        self.X = bf16(c["X"])
        self.mask = u8(c["mask"])
        self.ones = torch.ones_like(self.mask)
        self.Y = torch.empty_like(self.X)
        self.ws = torch.empty(wide.attn_proj_masked_workspace(self.T, m["d"], m["n_q"], m["n_kv"],
                                                              mode="decode", kv_cap=m["kv_cap"]),
                              dtype=torch.uint8, device="cuda")
        self.wide, self.i = wide, 0

    def step(self, ones=False):
        m = self.m
        Wq, Wk, Wv, Wo, Kc, Vc = self.sets[self.i % len(self.sets)]
        self.i += 1
        self.wide.attn_proj_masked(self.X, self.ones if ones else self.mask, Wq, Wk, Wv, Wo,
                                   n_q=m["n_q"], n_kv=m["n_kv"], mode="decode", K_cache=Kc,
                                   V_cache=Vc, kv_len=self.L, out=self.Y, workspace=self.ws)

    def work(self, ones=False):
        am = np.ones_like(self.c["mask"]) if ones else (self.c["mask"] != 0)
        return _attn_decode_bytes(self.m, am, self.m["d"], self.L)

    def oracle_sample(self, S):
        from oracle import attn_masked
        c, m = self.c, self.m
        t0 = time.perf_counter()
        attn_masked(c["X"][:S], c["mask"][:S], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                    n_kv=m["n_kv"], head_dim=HD, decode=True, K_cache=c["K_cache"][:S],
                    V_cache=c["V_cache"][:S], kv_len=self.L, dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


class AttnDecodeMaskedCache:
    """Llama-3.1-8B-shaped attention decode over masked caches: batch 16 at position 8192,
    where each (sequence, group) cache holds only the earlier tokens that kept the group
    (about half of 8192 at keep 4 of 8).  All-ones comparison: every group kept, every
    cache full (kv_len = position)."""

    def __init__(self, B=16, pos=8192):
        from synth.workloads import attn_case
        self.name = "attn_decode_masked_cache_8b"
        self.c = attn_case(self.name, B, keep=0.5, mask_kind="topk", decode=True, kv_len=pos,
                           kv_cap=pos + 1)
        m = self.c["meta"]
        self.m, self.T, self.pos = m, B, pos
        rng = np.random.default_rng(8192)
        self.lens = rng.binomial(pos, 0.5, size=(B, m["n_kv"])).astype(np.int32)
        self.config = dict(workload=self.name, B=B, position=pos, kv_cap=pos + 1,
                           mean_cache_len=round(float(self.lens.mean()), 1), d_model=m["d"],
                           n_q_heads=m["n_q"], n_kv_heads=m["n_kv"], head_dim=HD, keep=m["keep"],
                           masks="top-k")
        self.bound = "hbm"

    def upload(self, torch, wide, bf16, u8):
        c, m = self.c, self.m
        set_bytes = (2 * m["n_q"] + 2 * m["n_kv"]) * HD * m["d"] * 2 + 2 * c["K_cache"].size * 2
        self.sets = []
        for _ in range(_copies(set_bytes)):
            self.sets.append((bf16(c["Wq"]), bf16(c["Wk"]), bf16(c["Wv"]),
                              wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]), bf16(c["K_cache"]),
                              bf16(c["V_cache"])))
        self.X = bf16(c["X"])
        self.mask = u8(c["mask"])
        self.ones = torch.ones_like(self.mask)
        self.L = torch.from_numpy(self.lens).cuda()
        self.full = torch.full_like(self.L, self.pos)
        self.Y = torch.empty_like(self.X)
        self.ws = torch.empty(wide.attn_proj_masked_workspace(self.T, m["d"], m["n_q"], m["n_kv"],
                                                              mode="decode", kv_cap=self.pos + 1),
                              dtype=torch.uint8, device="cuda")
        self.wide, self.i = wide, 0

    def step(self, ones=False):
        m = self.m
        Wq, Wk, Wv, Wo, Kc, Vc = self.sets[self.i % len(self.sets)]
        self.i += 1
        self.wide.attn_decode_masked_cache(self.X, self.ones if ones else self.mask, Wq, Wk, Wv,
                                           Wo, n_q=m["n_q"], n_kv=m["n_kv"], K_cache=Kc,
                                           V_cache=Vc, kv_len=self.full if ones else self.L,
                                           pos=self.pos, out=self.Y, workspace=self.ws)

    def work(self, ones=False):
        am = np.ones_like(self.c["mask"]) if ones else (self.c["mask"] != 0)
        lens = np.full_like(self.lens, self.pos) if ones else self.lens
        w = _attn_decode_bytes(self.m, am, self.m["d"], 0)
        r = self.m["n_q"] // self.m["n_kv"]
        kept_len = float(((lens + 1) * am).sum())
        w["attn_core_decode"] = kept_len * 2 * HD * 2 + float(am.sum()) * r * HD * 2
        return w

    def oracle_sample(self, S):
        from oracle import attn_masked
        c, m = self.c, self.m
        t0 = time.perf_counter()
        attn_masked(c["X"][:S], c["mask"][:S], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                    n_kv=m["n_kv"], head_dim=HD, decode=True, K_cache=c["K_cache"][:S],
                    V_cache=c["V_cache"][:S], kv_len=self.lens[:S], pos=self.pos,
                    dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


class AttnDecodePaged(AttnDecodeMaskedCache):
    """AttnDecodeMaskedCache's caches and lengths held in a paged pool: pages of
    `page_size` slots dealt to the (sequence, group) caches in a seeded random order,
    one page table per pair."""

    def __init__(self, B=16, pos=8192, page_size=16):
        super().__init__(B, pos)
        m = self.m
        self.name = f"attn_decode_paged_8b_p{page_size}"
        self.ps = page_size
        self.max_pages = (pos + 1 + page_size - 1) // page_size
        self.n_pages = B * m["n_kv"] * self.max_pages
        perm = np.random.default_rng(page_size).permutation(self.n_pages)
        self.table = perm.reshape(B, m["n_kv"], self.max_pages).astype(np.int32)
        self.config.update(workload=self.name, kv_cap=self.max_pages * page_size,
                           page_size=page_size, pages_per_pair=self.max_pages,
                           pool_pages=self.n_pages, page_order="shuffled")

    def _pool(self, cache):
        B, n_kv, cap, _ = cache.shape
        pad = np.zeros((B, n_kv, self.max_pages * self.ps, HD), cache.dtype)
        pad[:, :, :cap] = cache
        pool = np.empty((self.n_pages, self.ps, HD), cache.dtype)
        pool[self.table.reshape(-1)] = pad.reshape(-1, self.ps, HD)
        return pool

    def upload(self, torch, wide, bf16, u8):
        super().upload(torch, wide, bf16, u8)
        c = self.c
        pools = self._pool(c["K_cache"]), self._pool(c["V_cache"])
        self.sets = [s[:4] + (bf16(pools[0]), bf16(pools[1])) for s in self.sets]
        self.pt = torch.from_numpy(self.table).cuda()
        m = self.m
        self.ws = torch.empty(wide.attn_proj_masked_workspace(
            self.T, m["d"], m["n_q"], m["n_kv"], mode="decode", kv_cap=self.max_pages * self.ps),
            dtype=torch.uint8, device="cuda")

    def step(self, ones=False):
        m = self.m
        Wq, Wk, Wv, Wo, Kp, Vp = self.sets[self.i % len(self.sets)]
        self.i += 1
        self.wide.attn_decode_masked_paged(self.X, self.ones if ones else self.mask, Wq, Wk, Wv,
                                           Wo, n_q=m["n_q"], n_kv=m["n_kv"], K_pool=Kp,
                                           V_pool=Vp, page_table=self.pt,
                                           kv_len=self.full if ones else self.L, pos=self.pos,
                                           out=self.Y, workspace=self.ws)

    def oracle_sample(self, S):
        from oracle import attn_masked, paged_to_contiguous
        c, m = self.c, self.m
        t0 = time.perf_counter()
        Kc, Vc, L = paged_to_contiguous(self._pool(c["K_cache"]), self._pool(c["V_cache"]),
                                        self.table[:S], self.lens[:S])
        attn_masked(c["X"][:S], c["mask"][:S], c["Wq"], c["Wk"], c["Wv"], c["Wo"], n_q=m["n_q"],
                    n_kv=m["n_kv"], head_dim=HD, decode=True, K_cache=Kc, V_cache=Vc,
                    kv_len=L, pos=self.pos, dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


class LayerDecode:
    """Llama-3.1-8B-shaped decoder layer, decode: batch 32 over an 8192-entry cache."""

    def __init__(self, B=32, L=8192, keep=0.5, kind="router", ffn_group=128, attn_keep=None):
        from synth.workloads import layer_8b
        self.name = layer_name("layer_decode_8b", keep, kind, ffn_group, attn_keep)
        self.c = layer_8b(B, decode=True, L=L, keep=keep, kind=kind, ffn_group=ffn_group,
                          attn_keep=attn_keep)
        m = self.c["meta"]
        self.m, self.T, self.L = m, B, L
        self.config = dict(workload=self.name, B=B, kv_len=L, d_model=m["d"], d_ff=m["F"],
                           n_ffn_groups=m["n_ffn"], n_q_heads=m["n_q"], n_kv_heads=m["n_kv"],
                           head_dim=HD, rope_theta=m["rope_theta"], keep=keep,
                           masks=f"{kind} top-k" if kind == "router" else kind,
                           **measured_keep(self.c))
        self.bound = "hbm"

    def upload(self, torch, wide, bf16, u8):
        c, m = self.c, self.m
        self.sets = []
        for _ in range(2):
            self.sets.append(dict(
                rms1=bf16(c["rms1"]), rms2=bf16(c["rms2"]), Wq=bf16(c["Wq"]), Wk=bf16(c["Wk"]),
                Wv=bf16(c["Wv"]), Wo_packed=wide.pack_kmajor(bf16(c["Wo"]), m["n_kv"]),
                W_gate=bf16(c["W_gate"]), W_up=bf16(c["W_up"]),
                W_down_packed=wide.pack_kmajor(bf16(c["W_down"]), m["n_ffn"]),
                K_cache=bf16(c["K_cache"]), V_cache=bf16(c["V_cache"])))
        self.X = bf16(c["X"])
        self.masks = (u8(c["attn_mask"]), u8(c["ffn_mask"]))
        self.ones = (torch.ones_like(self.masks[0]), torch.ones_like(self.masks[1]))
        self.Y = torch.empty_like(self.X)
        ws = wide.layer_masked_workspace(self.T, m["d"], m["F"], m["n_ffn"], m["n_q"], m["n_kv"],
                                         HD, m["rope_theta"], m["eps"], mode="decode",
                                         kv_cap=m["kv_cap"])
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.wide, self.i = wide, 0

    def step(self, ones=False):
        m = self.m
        S = self.sets[self.i % len(self.sets)]
        self.i += 1
        am, fm = self.ones if ones else self.masks
        self.wide.layer_masked(self.X, am, fm, S, n_q=m["n_q"], n_kv=m["n_kv"], head_dim=HD,
                               rope_theta=m["rope_theta"], eps=m["eps"], mode="decode",
                               K_cache=S["K_cache"], V_cache=S["V_cache"], kv_len=self.L,
                               out=self.Y, workspace=self.ws)

    def work(self, ones=False):
        m = self.m
        d, G, B = m["d"], m["F"] // m["n_ffn"], self.T
        am = np.ones_like(self.c["attn_mask"]) if ones else (self.c["attn_mask"] != 0)
        fm = np.ones_like(self.c["ffn_mask"]) if ones else (self.c["ffn_mask"] != 0)
        U, kept = float(fm.any(axis=0).sum()), float(fm.sum())
        w = _attn_decode_bytes(m, am, d, self.L)
        w["ffn_up_decode"] = U * 2 * G * d * 2 + B * d * 2 + kept * G * 2
        w["ffn_down_decode"] = U * G * d * 2 + kept * G * 2 + B * d * 2
        return w

    def oracle_sample(self, S):
        from oracle import layer_masked
        c, m = self.c, self.m
        W = {k: c[k] for k in ("rms1", "rms2", "Wq", "Wk", "Wv", "Wo", "W_gate", "W_up", "W_down")}
        t0 = time.perf_counter()
        layer_masked(c["X"][:S], c["attn_mask"][:S], c["ffn_mask"][:S], W, n_q=m["n_q"],
                     n_kv=m["n_kv"], head_dim=HD, n_ffn=m["n_ffn"], rope_theta=m["rope_theta"],
                     eps=m["eps"], decode=True, K_cache=c["K_cache"][:S], V_cache=c["V_cache"][:S],
                     kv_len=self.L, dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


class RouterPrefill:
    """The layer's FFN router on the GPU: logits X R^T and the top-k mask (56 of 112
    groups) for 8192 tokens of d_model 4096, with the mask's packed bit words."""

    def __init__(self, T=8192):
        import synth
        self.name, self.T, self.d, self.n, self.k = "router_prefill_8b", T, 4096, 112, 56
        self.X = synth.normal(self.name, "X", (T, self.d))
        self.R = synth.normal(self.name, "R", (self.n, self.d), std=self.d ** -0.5)
        self.config = dict(workload=self.name, T=T, d_model=self.d, n_groups=self.n, k=self.k,
                           router="linear, bf16, fp32 logits, top-k with ties to the lower group")
        self.bound = "hbm"

    def upload(self, torch, wide, bf16, u8):
        self.Xd, self.Rp = bf16(self.X), wide.pack_router(bf16(self.R))
        self.out = dict(mask=torch.empty((self.T, self.n), dtype=torch.uint8, device="cuda"),
                        packed=torch.empty((self.T, (self.n + 63) // 64), dtype=torch.int64,
                                           device="cuda"))
        self.wide = wide

    def step(self, ones=False):
        # all-ones: every group kept (k = n), the same logits work
        self.wide.router_topk(self.Xd, self.Rp, self.n if ones else self.k, self.n, out=self.out)

    def work(self, ones=False):
        T, d, n = self.T, self.d, self.n
        return {"router_topk": T * d * 2 + n * d * 2 + T * n + T * 8 * ((n + 63) // 64)}

    def oracle_sample(self, S):
        from oracle import router_topk
        t0 = time.perf_counter()
        router_topk(self.X[:S], self.R, self.k, dtype=ORACLE_DTYPE)
        return time.perf_counter() - t0


WORKLOADS = {"layer_prefill_8b": LayerPrefill, "ffn_prefill_3b": FfnPrefill,
             "attn_prefill_8b": AttnPrefill, "layer_decode_8b": LayerDecode,
             "attn_decode_8b": AttnDecode, "ffn_decode_8b_B1": lambda: FfnDecode(1),
             "ffn_decode_8b_B8": lambda: FfnDecode(8), "ffn_decode_8b_B32": lambda: FfnDecode(32),
             "ffn_decode_8b_B64": lambda: FfnDecode(64), "router_prefill_8b": RouterPrefill,
             "attn_decode_masked_cache_8b": AttnDecodeMaskedCache,
             "attn_decode_paged_8b_p16": lambda: AttnDecodePaged(page_size=16),
             "attn_decode_paged_8b_p128": lambda: AttnDecodePaged(page_size=128),
             "layer_prefill_8b_routed": LayerPrefillRouted,
             "layer_decode_masked_cache_8b": LayerDecodeMaskedCache}


# ------------------------------------------------------------- measurement

def warm(torch, fn, steps, min_s=0.3):
    """Untimed warm-up: at least `steps` steps and at least `min_s` seconds, so that
    the clocks have settled before a short (decode) step is timed."""
    t0 = time.perf_counter()
    n = 0
    while n < steps or time.perf_counter() - t0 < min_s:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timed(torch, fn, steps, stream):
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def graph_step(torch, W, ones=False):
    """The workload's step recorded into HIP graphs (torch.cuda.graph), one graph per
    input set, replayed in the same rotation, as a serving loop may launch a decode
    step.  Every call of a decode step writes the same cache slots from the same
    inputs, so a replay repeats the eager step."""
    # decode workloads rotate weight (and cache) sets; prefill ones use one set
    holder = getattr(W, "inner", W)
    n_sets = len(getattr(holder, "sets", [None]))
    fn = lambda: W.step(ones=ones)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager pass over the sets on a side stream first
        for _ in range(n_sets):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for _ in range(n_sets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs.append(g)
    torch.cuda.synchronize()
    k = [0]

    def replay():
        graphs[k[0] % len(graphs)].replay()
        k[0] += 1
    return replay


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source (its recorded hash must match)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in sorted(rec.get("sources", [])):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec.get("source_sha256"):
        return None
    return rec.get("bytes_per_launch")


def gemm_ceiling(torch):
    """Dense bf16 C = A B with torch.matmul (hipBLASLt) at the layer's FFN shapes, on operands
    with the workloads' scales (A ~ N(0, 1), B ~ N(0, 0.02)) and on zeros: the MFMA clock, and so
    the dense rate, depends on the power the operand values draw."""
    out = {"metric": "dense bf16 GEMM TFLOP/s (torch.matmul / hipBLASLt)", "peak": PEAK_BF16_TFLOPS,
           "shapes": []}
    gen = torch.Generator(device="cuda").manual_seed(0)
    for (M, N, K) in [(8192, 8192, 4096), (8192, 28672, 4096), (8192, 4096, 14336)]:
        row = {"M": M, "N": N, "K": K}
        for kind in ("random", "zeros"):
            if kind == "random":
                A = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
                B = (0.02 * torch.randn(K, N, device="cuda", generator=gen)).to(torch.bfloat16)
            else:
                A = torch.zeros(M, K, device="cuda", dtype=torch.bfloat16)
                B = torch.zeros(K, N, device="cuda", dtype=torch.bfloat16)
            stream = torch.cuda.current_stream()
            warm(torch, lambda: A @ B, 3)
            ms = timed(torch, lambda: A @ B, 10, stream)
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            row[kind] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
            del A, B
        out["shapes"].append(row)
    return out


def cpu_info():
    """CPU model (from /proc/cpuinfo) and the BLAS NumPy uses (threadpoolctl)."""
    model, blas = None, None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = f"{p.get('internal_api')} {p.get('version')}"
                break
    except Exception:  # pragma: no cover
        pass
    return model, blas


def c1_single_thread():
    """The oracle (fp32) on the tiny FFN configuration (64 tokens, d 256, d_ff 1024 in 16
    groups), one BLAS thread: tokens/s (median of 5)."""
    from threadpoolctl import threadpool_limits
    from oracle import ffn_masked
    from synth.workloads import tiny_ffn
    c = tiny_ffn()
    runs = []
    with threadpool_limits(1, "blas"):
        for _ in range(6):
            t0 = time.perf_counter()
            ffn_masked(c["X"], c["mask"], c["W_gate"], c["W_up"], c["W_down"], dtype=ORACLE_DTYPE)
            runs.append(time.perf_counter() - t0)
    return round(c["X"].shape[0] / float(np.median(runs[1:])), 1)


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else None
    except Exception:  # pragma: no cover
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="layer_prefill_8b", choices=sorted(WORKLOADS))
    ap.add_argument("--oracle-tokens", type=int, default=None,
                    help="tokens of the CPU oracle sample (default: all T tokens)")
    ap.add_argument("--no-oracle", action="store_true")
    ap.add_argument("--keep", type=float, default=0.5,
                    help="layer workloads: kept fraction of groups per token")
    ap.add_argument("--masks", default="router", choices=["router", "bernoulli", "clustered"],
                    help="layer workloads: mask structure")
    ap.add_argument("--attn-keep", type=float, default=None,
                    help="layer workloads: the attention mask's own keep ratio (--keep is then "
                         "the FFN's)")
    ap.add_argument("--sort-ffn", action="store_true",
                    help="layer prefill workloads: sort the tokens of the FFN down projection "
                         "by the pattern of their first 8 FFN groups (WIDE_FLAG_FFN_TOKEN_SORT)")
    ap.add_argument("--ffn-group", type=int, default=128,
                    help="layer workloads: channels per FFN group (d_ff 14336 = groups x this)")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="how the timed steps are launched: eager calls, or replays of HIP graphs "
                         "that recorded the calls (as a serving loop may run decode; measured "
                         "4-5 us per step slower than eager calls on the 8B decode workloads, "
                         "whose steps are GPU-bound)")
    ap.add_argument("--skip-ones", action="store_true",
                    help="skip the all-ones comparison (profiler runs: only masked launches)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of a workload, run 3 plain device copies of this many bytes "
                         "(calibrates the HBM traffic counters) and exit")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="instead of a workload, time the vendor dense bf16 GEMM (torch.matmul, "
                         "hipBLASLt) on random and on zero operands at the 8B FFN shapes, print "
                         "one JSON line and exit (the practical MFMA ceiling on these inputs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: it measures the single-GPU masked path "
              "(N > 1 is not supported).", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_wide_mask_amd as wide
    from synth import bf16_bits

    def bf16(a):
        """float32 array of bf16-exact values -> bf16 device tensor with the same bits"""
        bits = bf16_bits(np.asarray(a, np.float32))
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    wide.lib()

    if args.gemm_ceiling:
        print(json.dumps(gemm_ceiling(torch)), flush=True)
        return

    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").uniform_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n * 4} bytes 3 times")
        return

    log(f"generating {args.workload} inputs")
    if args.workload.startswith("layer_"):
        W = WORKLOADS[args.workload](keep=args.keep, kind=args.masks, ffn_group=args.ffn_group,
                                     attn_keep=args.attn_keep)
    elif args.workload == "ffn_prefill_3b":
        W = FfnPrefill(ffn_group=args.ffn_group)
    else:
        W = WORKLOADS[args.workload]()
    if args.sort_ffn:
        if not isinstance(W, LayerPrefill):
            raise SystemExit("--sort-ffn applies to the layer prefill workloads")
        W.sort_ffn = True
        W.name += "_sortffn"
        W.config.update(workload=W.name, ffn_token_sort=True)
    W.upload(torch, wide, bf16, u8)
    stream = torch.cuda.current_stream()
    graph = args.launch == "graph"

    warm(torch, W.step, args.warmup)
    ms_eager = None
    if graph:
        ms_eager = timed(torch, W.step, args.steps, stream)
        log(f"masked, eager calls: {ms_eager:.3f} ms/step")
        step = graph_step(torch, W)
        warm(torch, step, args.warmup)
    else:
        step = W.step

    # timed region: K masked steps as a caller runs them (no instrumentation)
    ms = timed(torch, step, args.steps, stream)
    log(f"masked: {ms:.3f} ms/step" + (" (graph replays)" if graph else ""))
    # the same K steps again, as eager calls, with a HIP event pair around every
    # kernel launch, on the launch's stream: per-kernel times for the roofline (the
    # events add a few microseconds per launch, so the step time above is taken
    # without them)
    wide.trace_reset()
    wide.trace_enable(True)
    ms_traced = timed(torch, W.step, args.steps, stream)
    wide.trace_enable(False)
    kern = wide.trace_collect()
    wide.trace_reset()
    log(f"masked, traced: {ms_traced:.3f} ms/step")

    # the same kernels, grid policy and inputs with all-ones masks
    ms_ones = None
    if not args.skip_ones:
        warm(torch, lambda: W.step(ones=True), args.warmup)
        # timed like the masked region (no instrumentation, the same launch kind)
        ones_step = graph_step(torch, W, ones=True) if graph else (lambda: W.step(ones=True))
        if graph:
            warm(torch, ones_step, args.warmup)
        ms_ones = timed(torch, ones_step, max(3, args.steps // 2), stream)
        log(f"all-ones: {ms_ones:.3f} ms/step")

    work = W.work()
    hbm = getattr(W, "bound", "mfma") == "hbm"
    scale, peak, unit = (1e9, PEAK_HBM_GBS, "GB/s") if hbm else (1e12, PEAK_BF16_TFLOPS, "TFLOP/s")
    per_kernel = {}
    for k, (n, tot) in sorted(kern.items(), key=lambda kv: -kv[1][1]):
        avg = tot / max(n, 1)
        e = dict(launches=n, avg_us=round(avg * 1e3, 2),
                 share=round(tot / (ms_traced * args.steps), 4))
        if k in work:
            rate = work[k] / (avg * 1e-3) / scale
            e["gbs" if hbm else "tflops"] = round(rate, 1)
            e["frac"] = round(rate / peak, 4)
        per_kernel[k] = e
    dominant = max((k for k in kern if k in work), key=lambda k: kern[k][1])
    n_dom, tot_dom = kern[dominant]
    achieved = work[dominant] / (tot_dom / n_dom * 1e-3) / scale
    total_work = sum(work.values())
    step_rate = total_work / (ms * 1e-3) / scale

    result = {
        "metric": METRIC,
        "value": round(W.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init weights, router/top-k masks)",
        "config": W.config,
        "roofline": {
            "bound": "hbm" if hbm else "mfma",
            "kernel": dominant,
            "achieved": round(achieved, 1),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic_from_profiles(dominant, W.name),
        },
        "step_roofline": {"unit": unit, "achieved": round(step_rate, 1),
                          "frac": round(step_rate / peak, 4),
                          "work": "touched bytes" if hbm else "active FLOPs"},
        "launch": "hip_graph" if graph else "eager",
        "eager_ms_per_step": round(ms_eager, 4) if ms_eager else None,
        "traced_ms_per_step": round(ms_traced, 4),
        "all_ones_ms_per_step": round(ms_ones, 4) if ms_ones else None,
        "speedup_vs_all_ones": round(ms_ones / ms, 3) if ms_ones else None,
        "kernels": per_kernel,
    }

    if not args.no_oracle:
        S = args.oracle_tokens or W.T
        log(f"timing the CPU oracle on {S} tokens")
        secs = W.oracle_sample(S)
        model, blas = cpu_info()
        result["cpu_baseline"] = {
            "value": round(S / secs, 2),
            "unit": "tokens/s",
            "cores": blas_threads() or len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"first {S} of {W.T} tokens of the same inputs, dense fp32 NumPy oracle "
                      f"({secs:.1f} s)",
            "cpu_model": model,
            "blas": blas,
            "tiny_ffn_single_thread_tokens_per_s": c1_single_thread(),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
