"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Every mutation below is a plausible slip in a transformer forward pass; the
test patches it into the oracle module, runs the pin suite and requires a
failure.  This shows the pins are strong enough to trust the oracle.
"""
import numpy as np
import pytest

from oracle import model as om
from tests import test_oracle_pins as pins

_orig = {name: getattr(om, name) for name in
         ["layer_norm", "gelu", "apply_rope", "rope_cos_sin", "causal_attention", "layer_forward",
          "embed_blocks", "prefix_from_context", "stack_forward", "output_logits", "logits_at",
          "local_inputs"]}


def ln_unbiased(x, g, b, eps):
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).sum(-1, keepdims=True) / (x.shape[-1] - 1)
    return (x - mu) / np.sqrt(var + eps) * g + b


def gelu_tanh(x):
    return 0.5 * x * (1 + np.tanh(np.sqrt(2 / np.pi) * (x + 0.044715 * x ** 3)))


def rope_interleaved(x, positions, base):
    d = x.shape[-1]
    cos, sin = _orig["rope_cos_sin"](positions, d, base)
    cos, sin = cos[None, :, None, :], sin[None, :, None, :]
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * cos - x2 * sin
    out[..., 1::2] = x2 * cos + x1 * sin
    return out


def rope_freq_slip(positions, d, base):
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.asarray(positions, np.float64)[:, None] * (base ** (-i / d))[None, :]
    return np.cos(ang), np.sin(ang)


def attn_strict_mask(q, k, v, q_pos, k_pos):
    # a key is visible only if strictly earlier, except position 0 which sees itself
    return _orig["causal_attention"](q, k, v, q_pos, np.where(np.asarray(k_pos) > 0, np.asarray(k_pos) + 1, k_pos))


def attn_scale_slip(q, k, v, q_pos, k_pos):
    return _orig["causal_attention"](q / np.sqrt(q.shape[-1]), k, v, q_pos, k_pos)


def layer_sequential(W, name, h, pos, n_heads, eps, base, cache=None, n_kv_heads=0, enc=None):
    # sequential residual: the MLP sees h + attn instead of h
    zero = {k: (np.zeros_like(v) if k.startswith(name + ".mlp") else v) for k, v in W.items()}
    h1 = _orig["layer_forward"](zero, name, h, pos, n_heads, eps, base, cache, n_kv_heads, enc)
    zero_attn = {k: (np.zeros_like(v) if k.startswith((name + ".attn", name + ".xattn")) else v)
                 for k, v in W.items()}
    return _orig["layer_forward"](zero_attn, name, h1, pos, n_heads, eps, base, None, n_kv_heads, enc)


def layer_no_qkv_bias(W, name, h, pos, n_heads, eps, base, cache=None, n_kv_heads=0, enc=None):
    W2 = dict(W)
    W2[f"{name}.attn.qkv.b"] = np.zeros_like(W[f"{name}.attn.qkv.b"])
    return _orig["layer_forward"](W2, name, h, pos, n_heads, eps, base, cache, n_kv_heads, enc)


def layer_gqa_interleaved(W, name, h, pos, n_heads, eps, base, cache=None, n_kv_heads=0, enc=None):
    # grouped-query slip: query head i uses key/value head i mod n_kv_heads instead of i // group
    hkv = n_kv_heads or n_heads
    if hkv == n_heads or enc is not None:
        return _orig["layer_forward"](W, name, h, pos, n_heads, eps, base, cache, n_kv_heads, enc)
    B, n, D = h.shape
    dh = D // n_heads
    a = om.layer_norm(h, W[f"{name}.ln1.g"], W[f"{name}.ln1.b"], eps)
    m = om.layer_norm(h, W[f"{name}.ln2.g"], W[f"{name}.ln2.b"], eps)
    qkv = a @ W[f"{name}.attn.qkv.w"] + W[f"{name}.attn.qkv.b"]
    q = om.apply_rope(qkv[..., :D].reshape(B, n, n_heads, dh), pos, base)
    k = om.apply_rope(qkv[..., D:D + hkv * dh].reshape(B, n, hkv, dh), pos, base)
    v = qkv[..., D + hkv * dh:].reshape(B, n, hkv, dh)
    if cache is not None:
        cache.append(k, v, pos)
        k, v, k_pos = cache.k, cache.v, cache.pos
    else:
        k_pos = np.asarray(pos)
    g = n_heads // hkv
    o = om.causal_attention(q, np.tile(k, (1, 1, g, 1)), np.tile(v, (1, 1, g, 1)), np.asarray(pos), k_pos)
    attn = o.reshape(B, n, D) @ W[f"{name}.attn.out.w"] + W[f"{name}.attn.out.b"]
    mlp = om.gelu(m @ W[f"{name}.mlp.up.w"] + W[f"{name}.mlp.up.b"]) @ W[f"{name}.mlp.down.w"] + W[f"{name}.mlp.down.b"]
    return h + attn + mlp


def layer_xattn_query_from_ln2(W, name, h, pos, n_heads, eps, base, cache=None, n_kv_heads=0, enc=None):
    # cross-attention queries normalised by LN2 (the MLP's LayerNorm) instead of LN1
    if enc is None:
        return _orig["layer_forward"](W, name, h, pos, n_heads, eps, base, cache, n_kv_heads, enc)
    base_out = _orig["layer_forward"](W, name, h, pos, n_heads, eps, base, cache, n_kv_heads, None)
    B, n, D = h.shape
    dh = D // n_heads
    hkv = n_kv_heads or n_heads
    m = om.layer_norm(h, W[f"{name}.ln2.g"], W[f"{name}.ln2.b"], eps)
    xq = (m @ W[f"{name}.xattn.q.w"] + W[f"{name}.xattn.q.b"]).reshape(B, n, n_heads, dh)
    xkv = enc @ W[f"{name}.xattn.kv.w"] + W[f"{name}.xattn.kv.b"]
    xk = np.repeat(xkv[..., :hkv * dh].reshape(B, -1, hkv, dh), n_heads // hkv, axis=2)
    xv = np.repeat(xkv[..., hkv * dh:].reshape(B, -1, hkv, dh), n_heads // hkv, axis=2)
    xo = om.cross_attention(xq, xk, xv).reshape(B, n, D)
    return base_out + xo @ W[f"{name}.xattn.out.w"] + W[f"{name}.xattn.out.b"]


def local_inputs_summand_shift(W, cfg, c, toks):
    # summation slip: slot i gets u_{i+1} (cyclically) instead of u_i
    z, enc = _orig["local_inputs"](W, cfg, c, toks)
    if cfg.context_mode != "sum":
        return z, enc
    u = om.prefix_from_context(W, cfg, c)
    return z - u[:, : z.shape[1]] + np.roll(u, -1, axis=1)[:, : z.shape[1]], enc


def local_inputs_zero_start(W, cfg, c, toks):
    # start slot left empty (zero vector) instead of the pad token's embedding
    z, enc = _orig["local_inputs"](W, cfg, c, toks)
    if cfg.context_mode == "prefix":
        return z, enc
    z = z.copy()
    z[:, 0] -= W["emb_token"][cfg.pad_id]
    return z, enc


def embed_reversed(W, cfg, tokens):
    B, S = tokens.shape
    L = cfg.block_len
    t = tokens.reshape(B, S // L, L)[:, :, ::-1].reshape(B, S)
    return _orig["embed_blocks"](W, cfg, t)


def prefix_transposed(W, cfg, c):
    u = c @ W["prefix.w"] + W["prefix.b"]
    return u.reshape(c.shape[0], cfg.d_model, cfg.prefix_len).transpose(0, 2, 1)


def stack_no_final_ln(W, prefix, n_layers, h, pos, n_heads, eps, base, caches=None, n_kv_heads=0, enc=None):
    # the token decoder's output skips its final LayerNorm
    if prefix != "tok":
        return _orig["stack_forward"](W, prefix, n_layers, h, pos, n_heads, eps, base, caches, n_kv_heads, enc)
    for l in range(n_layers):
        h = om.layer_forward(W, f"{prefix}.{l}", h, pos, n_heads, eps, base,
                             None if caches is None else caches[l], n_kv_heads, enc)
    return h


def logits_own_context(W, cfg, tokens, positions):
    # uses c_k (which has seen block k itself) instead of c_{k-1}
    L, P = cfg.block_len, cfg.prefix_len
    positions = list(positions)
    k_max = max(t // L for t in positions)
    padded = np.concatenate([tokens, np.zeros((tokens.shape[0], L), tokens.dtype)], 1)
    c = om.context_embeddings(W, cfg, padded, k_max + 1)
    out = []
    for t in positions:
        k, o = divmod(t, L)
        z = np.concatenate([om.prefix_from_context(W, cfg, c[:, k]),
                            W["emb_token"][tokens[:, k * L: k * L + o]]], 1)
        out.append(om.output_logits(W, om.token_decoder(W, cfg, z)[:, P - 1 + o]))
    return np.stack(out, 1)


def logits_slot_slip(W, cfg, tokens, positions):
    # reads the logits one slot late (slot P + o instead of P - 1 + o)
    L, P = cfg.block_len, cfg.prefix_len
    out = []
    for t in positions:
        k, o = divmod(t, L)
        c = om.context_embeddings(W, cfg, tokens, k)[:, k - 1]
        z = np.concatenate([om.prefix_from_context(W, cfg, c), W["emb_token"][tokens[:, k * L: k * L + o + 1]]], 1)
        out.append(om.output_logits(W, om.token_decoder(W, cfg, z)[:, P + o]))
    return np.stack(out, 1)


MUTATIONS = {
    "ln_unbiased_variance": ("layer_norm", ln_unbiased),
    "gelu_tanh_approximation": ("gelu", gelu_tanh),
    "rope_interleaved_pairs": ("apply_rope", rope_interleaved),
    "rope_frequency_exponent": ("rope_cos_sin", rope_freq_slip),
    "attention_mask_off_by_one": ("causal_attention", attn_strict_mask),
    "attention_scale_1_over_d": ("causal_attention", attn_scale_slip),
    "sequential_residual": ("layer_forward", layer_sequential),
    "missing_qkv_bias": ("layer_forward", layer_no_qkv_bias),
    "embedder_reversed_concat": ("embed_blocks", embed_reversed),
    "prefix_transposed_reshape": ("prefix_from_context", prefix_transposed),
    "token_decoder_final_ln_dropped": ("stack_forward", stack_no_final_ln),
    "context_of_own_block": ("logits_at", logits_own_context),
    "logit_slot_off_by_one": ("logits_at", logits_slot_slip),
    "gqa_heads_interleaved": ("layer_forward", layer_gqa_interleaved),
    "xattn_query_from_ln2": ("layer_forward", layer_xattn_query_from_ln2),
    "summand_index_shifted": ("local_inputs", local_inputs_summand_shift),
    "start_slot_zero": ("local_inputs", local_inputs_zero_start),
}

PIN_CALLS = [
    pins.test_layer_norm_matches_library,
    pins.test_gelu_closed_form_values,
    pins.test_rope_hand_example_and_pairing,
    pins.test_rope_matches_complex_rotation,
    pins.test_causal_attention_matches_library,
    pins.test_embedder_brute_force,
    lambda: pins.test_prefix_projection_layout(),
    lambda: pins.test_matches_library_crosscheck(dict()),
    lambda: pins.test_matches_library_crosscheck(dict(block_len=2, prefix_len=2)),
    lambda: pins.test_incremental_equals_full_recompute(dict(), 30, 13),
    pins.test_causality_bitwise,
    lambda: pins.test_grouped_query_attention_matches_library_and_incremental(2),
    lambda: pins.test_context_variants_match_library_crosscheck(dict(context_mode="sum", block_len=2)),
    lambda: pins.test_context_variants_match_library_crosscheck(dict(context_mode="xattn", prefix_len=2)),
]


def _run_pins():
    failures = 0
    for call in PIN_CALLS:
        try:
            call()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    return failures


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(om, attr, fn)
    assert _run_pins() > 0, f"no pin caught the planted mistake {mutation}"


def test_unmutated_oracle_passes_all_pins():
    assert _run_pins() == 0
