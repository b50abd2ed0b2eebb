"""An independent float64 Llama forward for pinning the reference decoder:
HuggingFace transformers' LlamaForCausalLM (the library that the GOTOken page
compares its engine with), loaded with the weights of a synthetic arena.

Test helper only; nothing in the product imports it.
"""
import numpy as np
import torch

import synth


def widen(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


def build(shape: synth.ModelShape, arena: np.ndarray, max_pos: int = 4096):
    from transformers import LlamaConfig, LlamaForCausalLM

    cfg = LlamaConfig(
        vocab_size=shape.vocab_size, hidden_size=shape.dim, intermediate_size=shape.hidden_dim,
        num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_heads,
        num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
        rms_norm_eps=float(np.float32(shape.norm_eps)), rope_theta=float(shape.rope_theta),
        tie_word_embeddings=bool(shape.tied_embeddings), max_position_embeddings=max_pos,
        attention_bias=False, mlp_bias=False, hidden_act="silu",
    )
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    try:
        model = LlamaForCausalLM(cfg)
    finally:
        torch.set_default_dtype(old)
    model.eval()
    v = synth.views(shape, arena)
    sd = {"model.embed_tokens.weight": v["token_emb"], "model.norm.weight": v["output_norm"]}
    names = {"wq": "self_attn.q_proj", "wk": "self_attn.k_proj", "wv": "self_attn.v_proj",
             "wo": "self_attn.o_proj", "w1": "mlp.gate_proj", "w3": "mlp.up_proj",
             "w2": "mlp.down_proj", "attn_norm": "input_layernorm",
             "ffn_norm": "post_attention_layernorm"}
    for l in range(shape.n_layers):
        for ours, theirs in names.items():
            sd[f"model.layers.{l}.{theirs}.weight"] = v[f"l{l}.{ours}"]
    sd["lm_head.weight"] = v["token_emb"] if shape.tied_embeddings else v["wcls"]
    with torch.no_grad():
        params = dict(model.named_parameters())
        for k, a in sd.items():
            if k in params:
                params[k].copy_(torch.from_numpy(widen(np.ascontiguousarray(a)).astype(np.float64)))
    return model


def logits(model, tokens) -> np.ndarray:
    """float64 logits [len(tokens)][V] of one causal forward over ``tokens``."""
    with torch.no_grad():
        out = model(input_ids=torch.tensor([list(map(int, tokens))]), use_cache=False)
    return out.logits[0].numpy()
