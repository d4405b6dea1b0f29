"""Host-side checks of the benchmark's cost model (no GPU): the algorithmic decode bytes and prefill
FLOPs that bench.py divides by the measured phase times.  They are checked against what does not
come from the cost model's own arithmetic: the parameter inventory of the weight blob
(bt_workloads.weight_specs, the layout the library packs), the cache entries the oracle's attention
reads during an incremental generation (its own counters), the closed form of a layer's parameter
count, and the byte breakdown of the prefill-heavy workload in the pages' cost terms (parameter
I/O of both decoders, block-KV I/O)."""
import numpy as np
import pytest

import bench
import bt_workloads as wl
from oracle import model as om


def _sizes(cfg):
    return {n: int(np.prod(s)) for n, s, _ in wl.weight_specs(cfg)}


VARIANTS = [dict(), dict(context_mode="sum"), dict(context_mode="xattn", prefix_len=2), dict(n_kv_heads=1),
            dict(block_len=2, prefix_len=2), dict(block_len=8, prompt_len=29)]


@pytest.mark.parametrize("kw", VARIANTS)
def test_layer_parameter_counts_match_the_weight_blob(kw):
    cfg = wl.get_config("c0_tiny", **kw)
    sz = _sizes(cfg)
    assert bench._layer_params(cfg) == sum(v for k, v in sz.items() if k.startswith("blk.0."))
    assert bench._layer_params(cfg, True) == sum(v for k, v in sz.items() if k.startswith("tok.0."))


def test_layer_parameter_closed_form():
    """Multi-head attention with a 4D MLP: 12 D^2 weights and 13 D biases and gains per layer."""
    cfg = wl.get_config("c1_prefill_heavy")
    D = cfg.d_model
    assert cfg.d_mlp == 4 * D and cfg.kv_heads == cfg.n_heads
    assert bench._layer_params(cfg) == 12 * D * D + 13 * D
    assert bench._layer_matmul_params(cfg) == 12 * D * D


@pytest.mark.parametrize("kw", VARIANTS)
def test_decode_bytes_match_the_oracles_reads(kw):
    """Block-KV bytes are the oracle's block-attention reads; local-KV bytes its token-step reads
    plus, per block step, the P prefix entries counted twice (the prefix pass writes and reads them);
    weight bytes the blob's tensors that each step multiplies or normalises with."""
    cfg = wl.get_config("c0_tiny", **kw)
    W = wl.make_weights(cfg)
    prompt = wl.make_prompt(cfg)
    st, lg = om.prefill(W, cfg, prompt)
    blk_reads = tok_reads = 0
    prev = om.greedy(lg)
    for g in range(1, cfg.gen_len):
        b0, l0 = st.kv_reads_block, st.kv_reads_local
        lg = om.decode_step(W, cfg, st, prev)
        blk_reads += st.kv_reads_block - b0
        if g % cfg.block_len:
            tok_reads += st.kv_reads_local - l0
        prev = om.greedy(lg)
    w = 4 if cfg.dtype == "fp32" else 2
    kv = 2 * cfg.kv_heads * cfg.d_head
    B, D, G = cfg.batch, cfg.d_model, cfg.gen_len
    n_blk = (G - 1) // cfg.block_len
    parts = bench.decode_bytes_parts(cfg)
    assert parts["block_kv"] == B * w * cfg.n_block_layers * kv * blk_reads
    assert parts["local_kv"] == B * w * cfg.n_token_layers * kv * (tok_reads + 2 * cfg.lead * n_blk)
    sz = _sizes(cfg)
    tok = sum(v for k, v in sz.items() if k.startswith("tok.0."))
    blk = sum(v for k, v in sz.items() if k.startswith("blk.0."))
    head = sz["tok.lnf.g"] + sz["tok.lnf.b"] + sz["head.w"]
    ctx = sz["blk.lnf.g"] + sz["blk.lnf.b"] + sz["prefix.w"] + sz["prefix.b"]
    assert parts["weights"] == w * ((G - 1) * (cfg.n_token_layers * tok + head) +
                                    n_blk * (cfg.n_block_layers * blk + ctx))
    assert parts["embeddings"] == B * w * D * (G - 1 + n_blk)
    assert bench.decode_bytes(cfg) == sum(parts.values())


def test_prefill_heavy_breakdown():
    """The prefill-heavy workload: token-decoder parameter I/O 20.6 GB, block-decoder parameter I/O
    2.7 GB, block-KV I/O 19.3 GB over its 127 decode steps; 2.95 TFLOP of prefill."""
    cfg = wl.get_config("c1_prefill_heavy")
    p = bench.decode_bytes_parts(cfg)
    D, V = cfg.d_model, cfg.vocab
    tok_w = 2 * 127 * (cfg.n_token_layers * (12 * D * D + 13 * D) + 2 * D + V * D)
    assert abs(tok_w / 1e9 - 20.6) < 0.05
    assert abs((p["weights"] - tok_w) / 1e9 - 2.7) < 0.05
    assert abs(p["block_kv"] / 1e9 - 19.3) < 0.05
    assert abs(bench.prefill_flops(cfg) / 1e12 - 2.95) < 0.005


def test_stored_decode_traffic_is_tied_to_workload_and_sources(tmp_path, monkeypatch):
    """The stored counter total is used only for the workload it was taken on and while every library
    source and the code-generation flags hash the same."""
    import json
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"workload": "c1_prefill_heavy", "traffic_bytes": 1.0, "dispatches": 1,
           "source_sha256_16": bench.all_sources_hash()}
    (tmp_path / "traffic_decode_steps.json").write_text(json.dumps(rec))
    assert bench.stored_decode_step_traffic("c1_prefill_heavy") is not None
    assert bench.stored_decode_step_traffic("c2_decode_heavy") is None
    rec["source_sha256_16"] = "0" * 16
    (tmp_path / "traffic_decode_steps.json").write_text(json.dumps(rec))
    assert bench.stored_decode_step_traffic("c1_prefill_heavy") is None


def test_trace_in_step_duration_is_read_from_the_committed_summary(tmp_path, monkeypatch):
    """The in-step average is the first column pair of the back-to-back table, matched by the
    (possibly truncated) kernel name."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "kernels_c1_prefill_heavy.txt").write_text(
        "# header\n  total_ms    pct   calls    avg_us    min_us    max_us  kernel\n"
        "in_step_calls in_step_avg_us b2b_calls b2b_avg_us  kernel\n"
        "         6678           5.21       370       5.02  _ZN2bt13k_gemm_skinnyILi4E\n"
        "         5376           6.21         0       0.00  _ZN2bt10k_attn_outILi4E\n")
    assert bench.trace_in_step_us("c1_prefill_heavy", "_ZN2bt13k_gemm_skinnyILi4ELi1E") == 5.21
    assert bench.trace_in_step_us("c1_prefill_heavy", "_ZN2bt10k_attn_outILi4ELi1E") == 6.21
    assert bench.trace_in_step_us("c1_prefill_heavy", "_ZN2bt11k_layernorm") is None
    assert bench.trace_in_step_us("c2_decode_heavy", "_ZN2bt13k_gemm_skinnyILi4ELi1E") is None


def test_code_hash_ignores_comments_but_not_code(tmp_path):
    """Stored counters stay valid across an edit of a source's comments and lapse with any change of
    its code (string literals that hold comment markers are code)."""
    a, b, c, d = (tmp_path / n for n in ("a.hip", "b.hip", "c.hip", "d.hip"))
    a.write_text('int f(int x) {  // scaled\n  return 2 * x; /* twice */\n}\nconst char* s = "a // b";\n')
    b.write_text('// header\nint f(int x) {\n\n  return 2 * x;\n}  \nconst char* s = "a // b";\n')
    c.write_text('int f(int x) {  // scaled\n  return 3 * x; /* twice */\n}\nconst char* s = "a // b";\n')
    d.write_text('int f(int x) {  // scaled\n  return 2 * x; /* twice */\n}\nconst char* s = "a ";\n')
    assert bench.code_text(str(a)) == bench.code_text(str(b))
    assert bench.code_text(str(a)) != bench.code_text(str(c))
    assert bench.code_text(str(a)) != bench.code_text(str(d))
