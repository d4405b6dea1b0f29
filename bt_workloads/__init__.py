"""Seeded synthetic workloads for the Block Transformer inference path.

This module is shared by the CPU oracle and the GPU path.  It holds shapes,
seeds and random draws only: none of the method's arithmetic lives here.

Shapes follow the block-transformer summary page ("Block Transformer:
Global-to-Local Language Modeling for Fast Inference"), §5 "Evaluation
Methodology" (prefill-heavy 2048/128 and decode-heavy 128/2048 workloads,
vocabulary 50,304) and the long-context 8K setting of §5 "Main Quantitative
Results".  Weights are random-init N(0, 0.02^2); prompts are uniform token ids.
The pages measure trained Pythia-style models on Pile text; these synthetic
inputs stand in for them at the same shapes (timing does not depend on values).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace, asdict
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "Config", "CONFIGS", "get_config", "weight_specs", "make_weights",
    "make_prompt", "round_bf16", "padded_len", "block_kv_capacity",
]


@dataclass(frozen=True)
class Config:
    """Model + workload shape of one Block Transformer inference run."""
    name: str
    dtype: str            # "fp32" or "bf16": storage type of weights and KV caches
    vocab: int
    d_model: int
    n_heads: int
    d_mlp: int
    n_block_layers: int
    n_token_layers: int
    block_len: int        # L_B
    prefix_len: int       # P
    batch: int
    prompt_len: int
    gen_len: int
    pad_id: int = 0
    ln_eps: float = 1e-5
    rope_base: float = 10000.0
    n_kv_heads: int = 0   # key/value heads of every attention layer (grouped-query); 0 = n_heads
    # how the context embedding reaches the token decoder: "prefix" (P prefix vectors in the local
    # sequence), "sum" (L_B vectors added to the token inputs) or "xattn" (P vectors as encoder
    # states of a cross-attention branch in every token-decoder layer)
    context_mode: str = "prefix"

    @property
    def d_head(self) -> int:
        return self.d_model // self.n_heads

    @property
    def kv_heads(self) -> int:
        return self.n_kv_heads or self.n_heads

    @property
    def d_emb(self) -> int:
        return self.d_model // self.block_len

    @property
    def n_ctx(self) -> int:
        """Vectors the context projection produces."""
        return self.block_len if self.context_mode == "sum" else self.prefix_len

    @property
    def lead(self) -> int:
        """Local slots before the block's first token: the P prefix vectors, or one start slot."""
        return self.prefix_len if self.context_mode == "prefix" else 1

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)

    def as_dict(self) -> dict:
        return asdict(self)


def padded_len(cfg: Config, T: int) -> int:
    """Prompt length after left padding to a whole number of blocks (>= L_B)."""
    L = cfg.block_len
    return max(L, -(-T // L) * L)


def block_kv_capacity(cfg: Config, T: int, G: int) -> int:
    """Block-KV entries needed per layer for a T-token prompt and G generated tokens."""
    return -(-(padded_len(cfg, T) + G) // cfg.block_len)


_D768 = dict(vocab=50304, d_model=768, n_heads=12, d_mlp=3072,
             n_block_layers=6, n_token_layers=6)

CONFIGS: Dict[str, Config] = {
    # tiny fp32 model: vocab 256, L_B=4, d=64 (16-dim token embeddings), 2+2 layers
    "c0_tiny": Config("c0_tiny", "fp32", vocab=256, d_model=64, n_heads=2, d_mlp=256,
                      n_block_layers=2, n_token_layers=2, block_len=4, prefix_len=1,
                      batch=2, prompt_len=32, gen_len=16),
    # prefill-heavy: 2048 prompt tokens, 128 generated, batch 64
    "c1_prefill_heavy": Config("c1_prefill_heavy", "bf16", **_D768, block_len=4, prefix_len=1,
                               batch=64, prompt_len=2048, gen_len=128),
    # decode-heavy: 128 prompt tokens, 2048 generated, batch 256
    "c2_decode_heavy": Config("c2_decode_heavy", "bf16", **_D768, block_len=4, prefix_len=1,
                              batch=256, prompt_len=128, gen_len=2048),
    # ~1.2B non-embedding parameters, balanced prefill/decode
    "c3_1p2b": Config("c3_1p2b", "bf16", vocab=50304, d_model=2048, n_heads=16, d_mlp=8192,
                      n_block_layers=12, n_token_layers=12, block_len=4, prefix_len=1,
                      batch=128, prompt_len=2048, gen_len=2048),
    # block-length sweep at the d=768 shapes, 8K prompts, prefix length 2
    "c4_lb1": Config("c4_lb1", "bf16", **_D768, block_len=1, prefix_len=2,
                     batch=32, prompt_len=8192, gen_len=512),
    "c4_lb2": Config("c4_lb2", "bf16", **_D768, block_len=2, prefix_len=2,
                     batch=32, prompt_len=8192, gen_len=512),
    "c4_lb8": Config("c4_lb8", "bf16", **_D768, block_len=8, prefix_len=2,
                     batch=32, prompt_len=8192, gen_len=512),
    # token-level (vanilla) transformers on the same kernels, at the d=768 width and the same total
    # depth (12 layers) as the Block Transformers above: n_token_layers = 0 with L_B = 1
    "v1_vanilla_prefill_heavy": Config("v1_vanilla_prefill_heavy", "bf16", vocab=50304, d_model=768, n_heads=12,
                                       d_mlp=3072, n_block_layers=12, n_token_layers=0, block_len=1,
                                       prefix_len=1, batch=64, prompt_len=2048, gen_len=128),
    "v2_vanilla_decode_heavy": Config("v2_vanilla_decode_heavy", "bf16", vocab=50304, d_model=768, n_heads=12,
                                      d_mlp=3072, n_block_layers=12, n_token_layers=0, block_len=1,
                                      prefix_len=1, batch=256, prompt_len=128, gen_len=2048),
    # variants the pages name as compatible: grouped-query (4 KV heads) and multi-query attention
    # in every layer, at the decode-heavy shapes
    "f4_gqa4_decode_heavy": Config("f4_gqa4_decode_heavy", "bf16", **_D768, block_len=4, prefix_len=1,
                                   batch=256, prompt_len=128, gen_len=2048, n_kv_heads=4),
    "f4_mqa_decode_heavy": Config("f4_mqa_decode_heavy", "bf16", **_D768, block_len=4, prefix_len=1,
                                  batch=256, prompt_len=128, gen_len=2048, n_kv_heads=1),
    # context injection by summation (L_B = 4 summands) and by cross-attention (2 encoder states)
    "f4_sum_decode_heavy": Config("f4_sum_decode_heavy", "bf16", **_D768, block_len=4, prefix_len=1,
                                  batch=256, prompt_len=128, gen_len=2048, context_mode="sum"),
    "f4_xattn_decode_heavy": Config("f4_xattn_decode_heavy", "bf16", **_D768, block_len=4, prefix_len=2,
                                    batch=256, prompt_len=128, gen_len=2048, context_mode="xattn"),
    # a context beyond 8K: 32768-token prompts (8192 prompt blocks at L_B = 4)
    "f4_long32k_lb4": Config("f4_long32k_lb4", "bf16", **_D768, block_len=4, prefix_len=2,
                             batch=8, prompt_len=32768, gen_len=256),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg


def _layer_specs(prefix: str, D: int, F: int, QKV: int) -> List[Tuple[str, Tuple[int, ...], str]]:
    """QKV = output width of attn.qkv: D query columns, then the key and the value columns of the
    key/value heads (D each without grouped-query attention)."""
    return [
        (f"{prefix}.ln1.g", (D,), "ln_gain"),
        (f"{prefix}.ln1.b", (D,), "ln_bias"),
        (f"{prefix}.attn.qkv.w", (D, QKV), "normal"),
        (f"{prefix}.attn.qkv.b", (QKV,), "normal"),
        (f"{prefix}.attn.out.w", (D, D), "normal"),
        (f"{prefix}.attn.out.b", (D,), "normal"),
        (f"{prefix}.ln2.g", (D,), "ln_gain"),
        (f"{prefix}.ln2.b", (D,), "ln_bias"),
        (f"{prefix}.mlp.up.w", (D, F), "normal"),
        (f"{prefix}.mlp.up.b", (F,), "normal"),
        (f"{prefix}.mlp.down.w", (F, D), "normal"),
        (f"{prefix}.mlp.down.b", (D,), "normal"),
    ]


def weight_specs(cfg: Config) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) of every parameter, in canonical order.

    Matrices are [in, out]; the three tables are [vocab, width].  The order is
    the canonical weight-blob order of the C-ABI (include/bt.h).
    """
    V, D, F, NC = cfg.vocab, cfg.d_model, cfg.d_mlp, cfg.n_ctx
    KVW = cfg.kv_heads * cfg.d_head
    QKV = D + 2 * KVW
    specs: List[Tuple[str, Tuple[int, ...], str]] = [("emb_block", (V, cfg.d_emb), "normal")]
    for l in range(cfg.n_block_layers):
        specs += _layer_specs(f"blk.{l}", D, F, QKV)
    specs += [("blk.lnf.g", (D,), "ln_gain"), ("blk.lnf.b", (D,), "ln_bias")]
    if cfg.n_token_layers == 0:
        # token-level (vanilla) transformer: no prefix, no token decoder
        return specs + [("head.w", (V, D), "normal")]
    specs += [("prefix.w", (D, NC * D), "normal"), ("prefix.b", (NC * D,), "normal"),
              ("emb_token", (V, D), "normal")]
    for l in range(cfg.n_token_layers):
        specs += _layer_specs(f"tok.{l}", D, F, QKV)
        if cfg.context_mode == "xattn":
            specs += [(f"tok.{l}.xattn.q.w", (D, D), "normal"), (f"tok.{l}.xattn.q.b", (D,), "normal"),
                      (f"tok.{l}.xattn.kv.w", (D, 2 * KVW), "normal"),
                      (f"tok.{l}.xattn.kv.b", (2 * KVW,), "normal"),
                      (f"tok.{l}.xattn.out.w", (D, D), "normal"), (f"tok.{l}.xattn.out.b", (D,), "normal")]
    specs += [("tok.lnf.g", (D,), "ln_gain"), ("tok.lnf.b", (D,), "ln_bias"),
              ("head.w", (V, D), "normal")]
    return specs


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Finite inputs only: the carry into the exponent cannot overflow 32 bits there.
    """
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return x


def _draw(cfg: Config, seed: int, i: int, shape, kind: str, ln_jitter: bool, std: float) -> np.ndarray:
    rng = np.random.default_rng([seed, i])
    if kind == "normal" or ln_jitter:
        a = rng.standard_normal(shape, dtype=np.float32)
        a *= np.float32(std)
        if kind == "ln_gain":
            a += np.float32(1.0)
    elif kind == "ln_gain":
        a = np.ones(shape, np.float32)
    else:
        a = np.zeros(shape, np.float32)
    return round_bf16(a) if cfg.dtype == "bf16" else a


def make_weights(cfg: Config, seed: int = 0, ln_jitter: bool = False,
                 std: float = 0.02) -> Dict[str, np.ndarray]:
    """Random-init parameters as float32 arrays (bf16-representable when cfg.dtype is bf16).

    Tensor #i of weight_specs() is drawn from numpy.random.default_rng([seed, i]).
    LayerNorm gains are 1 and biases 0, unless ``ln_jitter`` draws them as
    1 + N(0, std^2) and N(0, std^2) to exercise the affine part of LayerNorm.
    Tensors are drawn on a thread pool; each has its own generator, so the
    result does not depend on the scheduling.
    """
    specs = weight_specs(cfg)
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        arrays = list(ex.map(lambda t: _draw(cfg, seed, t[0], t[1][1], t[1][2], ln_jitter, std),
                             enumerate(specs)))
    return {name: a for (name, _, _), a in zip(specs, arrays)}


def make_prompt(cfg: Config, batch: int | None = None, T: int | None = None,
                seed: int = 0) -> np.ndarray:
    """Uniform random token ids in [0, vocab), int32 [batch, T]."""
    B = cfg.batch if batch is None else batch
    T = cfg.prompt_len if T is None else T
    rng = np.random.default_rng([seed, 1_000_003])
    return rng.integers(0, cfg.vocab, (B, T)).astype(np.int32)
