"""Plain CPU oracle of Block Transformer inference (numpy).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
bench.py's cpu_baseline leg may import this module.  The GPU path never calls
it and shares no code with it; the only common dependency is the seeded input
module ``bt_workloads`` (shapes and random draws, none of the arithmetic).

Everything here follows the block-transformer summary page "Block Transformer:
Global-to-Local Language Modeling for Fast Inference" (arXiv 2406.02657):

* §3.2 "Big-Picture Architecture": embedder -> block decoder -> context
  embedding -> prefix -> token decoder -> output classifier.
* §3.4 "The Embedder": lookup of L_B tokens in a V x (D/L_B) table,
  concatenated into one D-vector per block; prompts that are not whole blocks
  are left padded.
* §3.4 "The Block Decoder": a standard causal transformer over block
  embeddings, one context embedding per block position; the tokens of block
  i+1 are predicted from the context embedding of block i.
* §3.4 "The Token Decoder": Proj maps the context embedding to P prefix
  vectors of width D, prepended to the current block's tokens; causal
  self-attention restricted to prefix + current block.
* §5 "Evaluation Methodology": Pythia architecture; §6 "Limitation 5":
  Pythia's parallel residual.

Where the pages are silent the plainest reading is taken (all of them are
listed, with reasons, in the design notes of this repository):
  - parallel residual h + Attn(LN1 h) + MLP(LN2 h), final LN per decoder;
  - exact erf GELU, LayerNorm with biased variance and eps from the config;
  - rotary embedding on the full head width, rotate-half pairing (i, i+d/2),
    frequencies base^(-2i/d); block position = block index, token-decoder
    position = local slot (prefix slots first);
  - block k (k >= 1) is predicted from c_{k-1}; the token decoder input is
    [prefix_0..prefix_{P-1}, x_{kL}, .., x_{kL+L-2}] and slot P-1+o predicts
    x_{kL+o}; block 0 has no prediction;
  - every linear map has a bias except the output classifier; three separate
    tables (embedder, token embedding, classifier);
  - greedy decoding, ties to the lowest id.

Context injection variants (§3.4 "The Token Decoder", alternatives to prefix tokens: summation,
as in MEGABYTE, and cross-attention), selected by cfg.context_mode:
  - "prefix" (default): as above;
  - "sum": Proj maps c to L_B vectors u_0..u_{L-1}; the local sequence has no prefix slots; slot
    0 holds a start token (the embedding of pad_id) and slot i >= 1 the token x_{kL+i-1}, and
    u_i is added to slot i; slot i predicts x_{kL+i};
  - "xattn": the same start-token local sequence without u; Proj maps c to P vectors used as
    encoder states: every token-decoder layer gets a third parallel branch
    h + Attn(LN1 h) + XAttn(LN1 h, enc) + MLP(LN2 h), multi-head attention from the layer's
    queries to all P states, without rotary embedding or mask.

With n_token_layers = 0 (and L_B = 1) the same definitions describe a token-level
("vanilla") transformer: the block decoder runs over tokens and its final LayerNorm
output at position t-1 goes straight to the classifier to predict token t.  The pages
compare Block Transformers against such Pythia-style models (§5 Evaluation Methodology,
baselines).

Computation runs in the dtype of the weights handed in (float64 for the exact
checks, float32 for the large shapes).  No blocking, fusion or reordering
beyond the definitions: matmuls are numpy's.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
from scipy.special import erf

Weights = Dict[str, np.ndarray]

# ----------------------------------------------------------------------------
# elementary operations
# ----------------------------------------------------------------------------


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis: biased variance, affine gain and bias."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) with the Gaussian CDF written through erf."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def rope_cos_sin(positions: np.ndarray, d_head: int, base: float):
    """cos/sin of the rotary angles pos * base^(-2i/d), i < d/2, in float64."""
    i = np.arange(d_head // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / d_head)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate pairs (i, i + d/2) of x [B, n, H, d] by the angle of each position."""
    d = x.shape[-1]
    cos, sin = rope_cos_sin(positions, d, base)
    cos = cos.astype(x.dtype)[None, :, None, :]
    sin = sin.astype(x.dtype)[None, :, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v per head, key j visible to query i iff k_pos[j] <= q_pos[i].

    q [B, nq, H, d], k/v [B, nk, H, d] -> [B, nq, H, d].
    """
    d = q.shape[-1]
    qh = np.transpose(q, (0, 2, 1, 3))            # [B, H, nq, d]
    kh = np.transpose(k, (0, 2, 3, 1))            # [B, H, d, nk]
    vh = np.transpose(v, (0, 2, 1, 3))            # [B, H, nk, d]
    s = np.matmul(qh, kh) / np.sqrt(np.asarray(d, dtype=q.dtype))
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]   # [nq, nk]
    s = np.where(visible[None, None], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    o = np.matmul(p, vh)                           # [B, H, nq, d]
    return np.transpose(o, (0, 2, 1, 3))


def cross_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v per head with every key visible (no positions, no mask)."""
    return causal_attention(q, k, v, np.zeros(q.shape[1], np.int64), np.zeros(k.shape[1], np.int64))


# ----------------------------------------------------------------------------
# one transformer layer (shared form of block decoder and token decoder layers)
# ----------------------------------------------------------------------------


@dataclass
class LayerCache:
    """Rotated keys and values of one layer, [B, n, H, d], with their positions."""
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    pos: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))

    @property
    def length(self) -> int:
        return 0 if self.k is None else self.k.shape[1]

    def append(self, k: np.ndarray, v: np.ndarray, pos: np.ndarray) -> None:
        if self.k is None:
            self.k, self.v = k, v
        else:
            self.k = np.concatenate([self.k, k], axis=1)
            self.v = np.concatenate([self.v, v], axis=1)
        self.pos = np.concatenate([self.pos, np.asarray(pos, np.int64)])


def layer_forward(W: Weights, name: str, h: np.ndarray, pos: np.ndarray, n_heads: int,
                  eps: float, base: float, cache: Optional[LayerCache] = None,
                  n_kv_heads: int = 0, enc: Optional[np.ndarray] = None) -> np.ndarray:
    """h + Attn(LN1 h) + MLP(LN2 h) for h [B, n, D] at positions pos [n].

    With a cache, the new keys/values are appended first and the queries attend
    over everything cached (earlier positions plus the causal part of the new ones).
    With n_kv_heads < n_heads (grouped-query attention) the projection has n_kv_heads key and
    value heads, and query head i uses key/value head i // (n_heads / n_kv_heads); the cache
    holds the n_kv_heads heads.
    With encoder states enc [B, P, D] the layer adds a cross-attention branch: queries from LN1 h,
    keys and values from enc (n_kv_heads heads, grouped the same way), output projection.
    """
    B, n, D = h.shape
    dh = D // n_heads
    hkv = n_kv_heads or n_heads
    a = layer_norm(h, W[f"{name}.ln1.g"], W[f"{name}.ln1.b"], eps)
    m = layer_norm(h, W[f"{name}.ln2.g"], W[f"{name}.ln2.b"], eps)

    qkv = a @ W[f"{name}.attn.qkv.w"] + W[f"{name}.attn.qkv.b"]
    q = qkv[..., :D].reshape(B, n, n_heads, dh)
    k = qkv[..., D:D + hkv * dh].reshape(B, n, hkv, dh)
    v = qkv[..., D + hkv * dh:D + 2 * hkv * dh].reshape(B, n, hkv, dh)
    q = apply_rope(q, pos, base)
    k = apply_rope(k, pos, base)
    if cache is not None:
        cache.append(k, v, pos)
        k_all, v_all, k_pos = cache.k, cache.v, cache.pos
    else:
        k_all, v_all, k_pos = k, v, np.asarray(pos)
    group = n_heads // hkv
    k_all = np.repeat(k_all, group, axis=2)   # head i -> key/value head i // group
    v_all = np.repeat(v_all, group, axis=2)
    o = causal_attention(q, k_all, v_all, np.asarray(pos), k_pos).reshape(B, n, D)
    attn = o @ W[f"{name}.attn.out.w"] + W[f"{name}.attn.out.b"]

    u = gelu(m @ W[f"{name}.mlp.up.w"] + W[f"{name}.mlp.up.b"])
    mlp = u @ W[f"{name}.mlp.down.w"] + W[f"{name}.mlp.down.b"]
    out = h + attn + mlp
    if enc is not None:
        P = enc.shape[1]
        xq = (a @ W[f"{name}.xattn.q.w"] + W[f"{name}.xattn.q.b"]).reshape(B, n, n_heads, dh)
        xkv = enc @ W[f"{name}.xattn.kv.w"] + W[f"{name}.xattn.kv.b"]
        xk = xkv[..., :hkv * dh].reshape(B, P, hkv, dh)
        xv = xkv[..., hkv * dh:].reshape(B, P, hkv, dh)
        xo = cross_attention(xq, np.repeat(xk, group, axis=2), np.repeat(xv, group, axis=2)).reshape(B, n, D)
        out = out + xo @ W[f"{name}.xattn.out.w"] + W[f"{name}.xattn.out.b"]
    return out


def stack_forward(W: Weights, prefix: str, n_layers: int, h: np.ndarray, pos: np.ndarray,
                  n_heads: int, eps: float, base: float,
                  caches: Optional[List[LayerCache]] = None, n_kv_heads: int = 0,
                  enc: Optional[np.ndarray] = None) -> np.ndarray:
    """Run n_layers layers named ``{prefix}.{l}`` and the final LayerNorm ``{prefix}.lnf``."""
    for l in range(n_layers):
        h = layer_forward(W, f"{prefix}.{l}", h, pos, n_heads, eps, base,
                          None if caches is None else caches[l], n_kv_heads, enc)
    return layer_norm(h, W[f"{prefix}.lnf.g"], W[f"{prefix}.lnf.b"], eps)


# ----------------------------------------------------------------------------
# the three components
# ----------------------------------------------------------------------------


def pad_prompt(cfg, prompt: np.ndarray) -> np.ndarray:
    """Left-pad each row with pad_id to a whole number of blocks (at least one block)."""
    B, T = prompt.shape
    L = cfg.block_len
    Tp = max(L, -(-T // L) * L)
    out = np.full((B, Tp), cfg.pad_id, dtype=np.int64)
    out[:, Tp - T:] = prompt
    return out


def embed_blocks(W: Weights, cfg, tokens: np.ndarray) -> np.ndarray:
    """Embedder: tokens [B, n*L_B] -> [B, n, D], block i = concat of its L_B table rows."""
    B, S = tokens.shape
    L = cfg.block_len
    assert S % L == 0
    rows = W["emb_block"][tokens]                  # [B, S, D/L_B]
    return rows.reshape(B, S // L, L * rows.shape[-1])


def block_decoder(W: Weights, cfg, e: np.ndarray, first_pos: int = 0,
                  caches: Optional[List[LayerCache]] = None) -> np.ndarray:
    """Block decoder: causal transformer over block embeddings -> context embeddings c."""
    pos = np.arange(first_pos, first_pos + e.shape[1])
    return stack_forward(W, "blk", cfg.n_block_layers, e, pos, cfg.n_heads,
                         cfg.ln_eps, cfg.rope_base, caches, getattr(cfg, "n_kv_heads", 0))


def prefix_from_context(W: Weights, cfg, c: np.ndarray) -> np.ndarray:
    """Proj: c [B, D] -> n_ctx vectors [B, n_ctx, D] (P prefix vectors, L_B summands with
    summation); vector j is slice [jD, (j+1)D)."""
    u = c @ W["prefix.w"] + W["prefix.b"]
    return u.reshape(c.shape[0], cfg.n_ctx, cfg.d_model)


def local_inputs(W: Weights, cfg, c: np.ndarray, toks: np.ndarray):
    """Token-decoder input of one block from the previous block's context embedding c [B, D] and
    the block's tokens toks [B, o] before the predicted one: (z [B, lead + o, D], encoder states
    or None).  Slot lead - 1 + o predicts the block's token o."""
    ctx = prefix_from_context(W, cfg, c)
    emb = W["emb_token"][toks]
    if cfg.context_mode == "prefix":
        return np.concatenate([ctx, emb], axis=1), None
    start = np.broadcast_to(W["emb_token"][cfg.pad_id], (c.shape[0], 1, cfg.d_model))
    z = np.concatenate([start, emb], axis=1)
    if cfg.context_mode == "sum":
        return z + ctx[:, : z.shape[1]], None
    assert cfg.context_mode == "xattn"
    return z, ctx


def token_decoder(W: Weights, cfg, z: np.ndarray, first_pos: int = 0,
                  caches: Optional[List[LayerCache]] = None, enc: Optional[np.ndarray] = None) -> np.ndarray:
    """Token decoder over the local sequence z [B, m, D] at local slots first_pos.. -> LN_f output."""
    pos = np.arange(first_pos, first_pos + z.shape[1])
    return stack_forward(W, "tok", cfg.n_token_layers, z, pos, cfg.n_heads,
                         cfg.ln_eps, cfg.rope_base, caches, getattr(cfg, "n_kv_heads", 0), enc)


def output_logits(W: Weights, y: np.ndarray) -> np.ndarray:
    """Output classifier, no bias: y [..., D] -> [..., V]."""
    return y @ W["head.w"].T


def greedy(logits: np.ndarray) -> np.ndarray:
    """argmax over the vocabulary; np.argmax returns the first (lowest) id on ties."""
    return np.argmax(logits, axis=-1)


# ----------------------------------------------------------------------------
# full recompute (teacher forced)
# ----------------------------------------------------------------------------


def context_embeddings(W: Weights, cfg, tokens: np.ndarray, n_blocks: int) -> np.ndarray:
    """c_0 .. c_{n_blocks-1} [B, n_blocks, D] of the padded sequence ``tokens``."""
    L = cfg.block_len
    return block_decoder(W, cfg, embed_blocks(W, cfg, tokens[:, : n_blocks * L]))


def is_vanilla(cfg) -> bool:
    """Token-level transformer: no token decoder, one token per block."""
    return cfg.n_token_layers == 0


def logits_at(W: Weights, cfg, tokens: np.ndarray, positions: Sequence[int]) -> np.ndarray:
    """Logits predicting token t from tokens[:, :t], for each t in positions.

    ``tokens`` [B, S] is a block-aligned sequence (padded prompt followed by
    generated ids); t ranges over [L_B, S].  Block k = t // L_B is decoded from
    c_{k-1} and the tokens of block k before t.  Returns [B, len(positions), V].
    """
    L, lead = cfg.block_len, cfg.lead
    positions = [int(t) for t in positions]
    assert all(L <= t <= tokens.shape[1] for t in positions)
    k_max = max(t // L for t in positions)
    c = context_embeddings(W, cfg, tokens, k_max)
    if is_vanilla(cfg):
        assert L == 1
        return np.stack([output_logits(W, c[:, t - 1]) for t in positions], axis=1)
    out = np.empty((tokens.shape[0], len(positions), W["head.w"].shape[0]), dtype=c.dtype)
    by_block: Dict[int, List[int]] = {}
    for idx, t in enumerate(positions):
        by_block.setdefault(t // L, []).append(idx)
    for k, idxs in by_block.items():
        o_max = max(positions[i] % L for i in idxs)
        z, enc = local_inputs(W, cfg, c[:, k - 1], tokens[:, k * L: k * L + o_max])
        y = token_decoder(W, cfg, z, enc=enc)
        for i in idxs:
            out[:, i] = output_logits(W, y[:, lead - 1 + positions[i] % L])
    return out


# ----------------------------------------------------------------------------
# incremental inference: prefill, then one token per decode step
# ----------------------------------------------------------------------------


@dataclass
class State:
    """Caches and counters of an incremental generation."""
    block_caches: List[LayerCache]
    local_caches: List[LayerCache]
    n_blocks: int                 # block-KV entries per layer
    generated: List[np.ndarray]   # ids emitted so far, each [B]
    kv_reads_block: int = 0       # block-KV entries read by attention (per row, per layer)
    kv_reads_local: int = 0       # local-KV entries read by attention (per row, per layer)
    summands: Optional[np.ndarray] = None   # "sum": u_0..u_{L-1} of the current block [B, L, D]
    enc: Optional[np.ndarray] = None        # "xattn": encoder states of the current block [B, P, D]

    @property
    def block_kv_len(self) -> int:
        return self.block_caches[0].length

    @property
    def local_kv_len(self) -> int:
        return self.local_caches[0].length if self.local_caches else 0


def _new_prefix_pass(W: Weights, cfg, st: State, c_last: np.ndarray) -> np.ndarray:
    """Reset the local caches, run the token decoder on the lead slots (P prefix vectors, or the
    start slot), return the logits of the last one.
    (Token-level transformer: the context embedding goes straight to the classifier.)"""
    if is_vanilla(cfg):
        return output_logits(W, c_last)
    lead = cfg.lead
    st.local_caches = [LayerCache() for _ in range(cfg.n_token_layers)]
    z, st.enc = local_inputs(W, cfg, c_last, np.zeros((c_last.shape[0], 0), np.int64))
    st.summands = prefix_from_context(W, cfg, c_last) if cfg.context_mode == "sum" else None
    y = token_decoder(W, cfg, z, 0, st.local_caches, st.enc)
    st.kv_reads_local += lead * (lead + 1) // 2
    return output_logits(W, y[:, lead - 1])


def prefill(W: Weights, cfg, prompt: np.ndarray):
    """Prefill: block decoder over every prompt block (filling the block KV), then the
    token decoder over the prefix of the last block's context only.  Returns (state, logits of token 0)."""
    x = pad_prompt(cfg, prompt)
    n0 = x.shape[1] // cfg.block_len
    st = State([LayerCache() for _ in range(cfg.n_block_layers)], [], n0, [])
    c = block_decoder(W, cfg, embed_blocks(W, cfg, x), 0, st.block_caches)
    st.kv_reads_block += n0 * (n0 + 1) // 2
    return st, _new_prefix_pass(W, cfg, st, c[:, -1])


def decode_step(W: Weights, cfg, st: State, prev: np.ndarray) -> np.ndarray:
    """Feed back the previous id and return the logits of the next token."""
    L, lead = cfg.block_len, cfg.lead
    st.generated.append(np.asarray(prev, dtype=np.int64))
    g = len(st.generated)                 # index of the token being predicted
    j = g % L                             # its offset within its block
    if j == 0:
        # the previous L_B generated ids complete a block: one block-decoder step
        blk = np.stack(st.generated[-L:], axis=1)                  # [B, L_B]
        e = embed_blocks(W, cfg, blk)                               # [B, 1, D]
        n = st.block_kv_len
        c = block_decoder(W, cfg, e, n, st.block_caches)
        st.kv_reads_block += n + 1
        st.n_blocks += 1
        return _new_prefix_pass(W, cfg, st, c[:, -1])
    # token step at local slot lead + j - 1
    z = W["emb_token"][st.generated[-1]][:, None, :]
    if cfg.context_mode == "sum":
        z = z + st.summands[:, j: j + 1]
    y = token_decoder(W, cfg, z, lead + j - 1, st.local_caches, st.enc)
    st.kv_reads_local += lead + j
    return output_logits(W, y[:, -1])


def generate(W: Weights, cfg, prompt: np.ndarray, G: int, keep_logits: bool = False,
             forced: Optional[np.ndarray] = None):
    """Greedy generation of G tokens: 1 prefill + (G-1) decode steps.

    With ``forced`` [B, G] the given ids are fed back instead of the argmax
    (teacher forcing on another run's id stream).  Returns (ids [B, G],
    logits [B, G, V] or None, state).
    """
    st, lg = prefill(W, cfg, prompt)
    ids, logits = [], []
    for g in range(G):
        if g > 0:
            lg = decode_step(W, cfg, st, ids[-1])
        if keep_logits:
            logits.append(lg)
        ids.append(greedy(lg) if forced is None else np.asarray(forced[:, g], np.int64))
    return (np.stack(ids, axis=1), np.stack(logits, axis=1) if keep_logits else None, st)


def weights_as(W: Weights, dtype) -> Weights:
    """Copy of the parameter dict in ``dtype`` (float64 for the exact checks)."""
    return {k: np.asarray(v, dtype=dtype) for k, v in W.items()}
