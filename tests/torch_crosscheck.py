"""An independent CPU formulation of the Block Transformer, built from torch's
library routines (layer_norm, scaled_dot_product_attention, gelu, linear) and a
complex-number rotary embedding.  It is used only to cross-check the numpy
oracle; it shares no code with it.

It follows the same pages ("Block Transformer: Global-to-Local Language Modeling
for Fast Inference", §3.2 and §3.4): a concatenating embedder, a causal block
decoder, a prefix projection and a causal token decoder over [prefix, block];
and the two context-injection alternatives of §3.4 "The Token Decoder": summation
(L_B projected vectors added to a start-token-led local sequence) and cross-attention
(P projected vectors as encoder states, attended from every token-decoder layer).
"""
from __future__ import annotations

import torch
import torch.nn.functional as F


def _t(a):
    return torch.as_tensor(a, dtype=torch.float64)


def rope_complex(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """x [B, H, n, d]: rotate the complex numbers x_i + 1j*x_{i+d/2} by exp(1j*pos*base^(-2i/d))."""
    d = x.shape[-1]
    z = torch.complex(x[..., : d // 2], x[..., d // 2:])
    freqs = base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(len(pos), d // 2, dtype=torch.float64),
                      pos.to(torch.float64)[:, None] * freqs[None, :])
    z = z * rot
    return torch.cat([z.real, z.imag], dim=-1)


def layer(W, name, h, pos, n_heads, eps, base, n_kv_heads=0, enc=None):
    B, n, D = h.shape
    dh = D // n_heads
    hkv = n_kv_heads or n_heads
    a = F.layer_norm(h, (D,), _t(W[f"{name}.ln1.g"]), _t(W[f"{name}.ln1.b"]), eps)
    m = F.layer_norm(h, (D,), _t(W[f"{name}.ln2.g"]), _t(W[f"{name}.ln2.b"]), eps)
    qkv = F.linear(a, _t(W[f"{name}.attn.qkv.w"]).T, _t(W[f"{name}.attn.qkv.b"]))
    q, k, v = qkv.split([D, hkv * dh, hkv * dh], dim=-1)
    heads = lambda t, nh: t.reshape(B, n, nh, dh).transpose(1, 2)   # noqa: E731
    q, k, v = heads(q, n_heads), heads(k, hkv), heads(v, hkv)
    q, k = rope_complex(q, pos, base), rope_complex(k, pos, base)
    # grouped-query attention through the library's own option (query heads share key/value heads)
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=hkv != n_heads)
    o = o.transpose(1, 2).reshape(B, n, D)
    attn = F.linear(o, _t(W[f"{name}.attn.out.w"]).T, _t(W[f"{name}.attn.out.b"]))
    u = F.gelu(F.linear(m, _t(W[f"{name}.mlp.up.w"]).T, _t(W[f"{name}.mlp.up.b"])), approximate="none")
    mlp = F.linear(u, _t(W[f"{name}.mlp.down.w"]).T, _t(W[f"{name}.mlp.down.b"]))
    out = h + attn + mlp
    if enc is not None:
        # cross-attention: no mask, no rotary; the queries share the self-attention's LayerNorm
        xq = heads(F.linear(a, _t(W[f"{name}.xattn.q.w"]).T, _t(W[f"{name}.xattn.q.b"])), n_heads)
        xk, xv = F.linear(enc, _t(W[f"{name}.xattn.kv.w"]).T, _t(W[f"{name}.xattn.kv.b"])).split(
            [hkv * dh, hkv * dh], dim=-1)
        P = enc.shape[1]
        xk = xk.reshape(B, P, hkv, dh).transpose(1, 2)
        xv = xv.reshape(B, P, hkv, dh).transpose(1, 2)
        xo = F.scaled_dot_product_attention(xq, xk, xv, enable_gqa=hkv != n_heads)
        out = out + F.linear(xo.transpose(1, 2).reshape(B, n, D), _t(W[f"{name}.xattn.out.w"]).T,
                             _t(W[f"{name}.xattn.out.b"]))
    return out


def stack(W, pre, n_layers, h, cfg, enc=None):
    pos = torch.arange(h.shape[1])
    for l in range(n_layers):
        h = layer(W, f"{pre}.{l}", h, pos, cfg.n_heads, cfg.ln_eps, cfg.rope_base, getattr(cfg, "n_kv_heads", 0),
                  enc)
    return F.layer_norm(h, (cfg.d_model,), _t(W[f"{pre}.lnf.g"]), _t(W[f"{pre}.lnf.b"]), cfg.ln_eps)


def block_logits(W, cfg, tokens, k):
    """Logits [B, L_B, V] for the L_B tokens of block k >= 1 of ``tokens`` [B, S] (teacher forced)."""
    L, P, D = cfg.block_len, cfg.prefix_len, cfg.d_model
    x = torch.as_tensor(tokens, dtype=torch.long)
    B = x.shape[0]
    e = _t(W["emb_block"])[x[:, : k * L]].reshape(B, k, D)
    c = stack(W, "blk", cfg.n_block_layers, e, cfg)[:, k - 1]
    proj = F.linear(c, _t(W["prefix.w"]).T, _t(W["prefix.b"]))
    toks = _t(W["emb_token"])[x[:, k * L: k * L + L - 1]]
    mode = getattr(cfg, "context_mode", "prefix")
    if mode == "prefix":
        z = torch.cat([proj.reshape(B, P, D), toks], dim=1)
        y = stack(W, "tok", cfg.n_token_layers, z, cfg)[:, P - 1:]
    else:
        # local sequence [start, x_kL .. x_kL+L-2], start = the pad token's embedding
        start = _t(W["emb_token"])[torch.full((B, 1), cfg.pad_id, dtype=torch.long)]
        z = torch.cat([start, toks], dim=1)
        if mode == "sum":
            y = stack(W, "tok", cfg.n_token_layers, z + proj.reshape(B, L, D), cfg)
        else:
            y = stack(W, "tok", cfg.n_token_layers, z, cfg, enc=proj.reshape(B, P, D))
    return (y @ _t(W["head.w"]).T).numpy()


def vanilla_logits(W, cfg, tokens, t):
    """Token-level transformer: logits [B, V] predicting token t from tokens[:, :t]."""
    x = torch.as_tensor(tokens[:, :t], dtype=torch.long)
    h = stack(W, "blk", cfg.n_block_layers, _t(W["emb_block"])[x], cfg)
    return (h[:, -1] @ _t(W["head.w"]).T).numpy()
