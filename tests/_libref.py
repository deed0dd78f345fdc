"""Independent library formulations used to pin the oracle (tests only).

These use torch's scaled_dot_product_attention / rms_norm / silu and the
transformers Llama implementation (rotary embedding, decoder layer), all in
float64 on the CPU.  They share no code with the oracle.
"""
import numpy as np
import torch
from transformers import LlamaConfig
from transformers.models.llama import modeling_llama as ml

F64 = torch.float64


def t64(a):
    return torch.as_tensor(np.asarray(a, np.float64))


def llama_config(d, F, n_q, n_kv, hd, theta, eps):
    cfg = LlamaConfig(hidden_size=d, intermediate_size=F, num_attention_heads=n_q,
                      num_key_value_heads=n_kv, head_dim=hd, rms_norm_eps=eps,
                      rope_theta=theta, attention_bias=False, mlp_bias=False,
                      max_position_embeddings=1 << 16)
    cfg._attn_implementation = "eager"
    return cfg


def rope_lib(x, pos, theta):
    """x [T, heads, hd] -> roped with transformers' Llama rotary embedding."""
    x = t64(x)
    T, H, hd = x.shape
    cfg = llama_config(hd * H, 4 * hd, H, H, hd, theta, 1e-5)
    rot = ml.LlamaRotaryEmbedding(cfg).to(F64)
    pos = torch.as_tensor(np.asarray(pos), dtype=torch.long)[None]
    cos, sin = rot(x[None].transpose(1, 2), pos)
    q = x[None].transpose(1, 2)                                    # [1, H, T, hd]
    q2, _ = ml.apply_rotary_pos_emb(q, q, cos, sin, unsqueeze_dim=1)
    return q2[0].transpose(0, 1).numpy()


def qkv_lib(X, Wq, Wk, Wv, n_q, n_kv, hd, theta, pos):
    X, Wq, Wk, Wv = (t64(a) for a in (X, Wq, Wk, Wv))
    T = X.shape[0]
    q = (X @ Wq.T).reshape(T, n_q, hd).numpy()
    k = (X @ Wk.T).reshape(T, n_kv, hd).numpy()
    v = (X @ Wv.T).reshape(T, n_kv, hd).numpy()
    if theta:
        q, k = rope_lib(q, pos, theta), rope_lib(k, pos, theta)
    return q, k, v


def sdpa(q, k, v, causal):
    """q [Tq, Hq, hd], k/v [Tk, Hkv, hd]; GQA by repeat_interleave of KV heads."""
    q, k, v = t64(q), t64(k), t64(v)
    r = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(r, dim=1)
    v = v.repeat_interleave(r, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1)[None], k.transpose(0, 1)[None], v.transpose(0, 1)[None], is_causal=causal)
    return o[0].transpose(0, 1).numpy()                           # [Tq, Hq, hd]


def llama_layer(X, W, n_q, n_kv, hd, theta, eps, part="layer"):
    """Dense transformers LlamaDecoderLayer (float64) with the given weights, causal.
    part="attn": x + self_attn(input_layernorm(x)) only; part="mlp":
    x + mlp(post_attention_layernorm(x)) only (each sublayer of the library layer
    with its residual, on the layer input)."""
    T, d = X.shape
    F = W["W_gate"].shape[0]
    cfg = llama_config(d, F, n_q, n_kv, hd, theta, eps)
    layer = ml.LlamaDecoderLayer(cfg, layer_idx=0).to(F64)
    sd = {
        "self_attn.q_proj.weight": t64(W["Wq"]), "self_attn.k_proj.weight": t64(W["Wk"]),
        "self_attn.v_proj.weight": t64(W["Wv"]), "self_attn.o_proj.weight": t64(W["Wo"]).T,
        "mlp.gate_proj.weight": t64(W["W_gate"]), "mlp.up_proj.weight": t64(W["W_up"]),
        "mlp.down_proj.weight": t64(W["W_down"]).T, "input_layernorm.weight": t64(W["rms1"]),
        "post_attention_layernorm.weight": t64(W["rms2"]),
    }
    layer.load_state_dict({k: v.contiguous() for k, v in sd.items()})
    rot = ml.LlamaRotaryEmbedding(cfg).to(F64)
    x = t64(X)[None]
    pos = torch.arange(T)[None]
    cos, sin = rot(x, pos)
    mask = torch.full((T, T), float("-inf"), dtype=F64).triu(1)[None, None]
    with torch.no_grad():
        if part == "attn":
            a = layer.self_attn(layer.input_layernorm(x), attention_mask=mask,
                                position_embeddings=(cos, sin))[0]
            return (x + a)[0].numpy()
        if part == "mlp":
            return (x + layer.mlp(layer.post_attention_layernorm(x)))[0].numpy()
        y = layer(x, attention_mask=mask, position_ids=pos, position_embeddings=(cos, sin))
    y = y[0] if isinstance(y, tuple) else y
    return y[0].numpy()
