"""Pins of the numpy oracle against facts fixed outside it: library routines,
closed forms, brute force, the invariants the pages state, and the numbers the
pages print (tests/golden/cost_model.json).

Page references are to "Block Transformer: Global-to-Local Language Modeling
for Fast Inference" (arXiv 2406.02657), summary page sections.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import bt_workloads as wl
from oracle import model as om
from tests import torch_crosscheck as tc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(**kw):
    return wl.get_config("c0_tiny", **kw)


def w64(cfg, seed=0, ln_jitter=True):
    return om.weights_as(wl.make_weights(cfg, seed=seed, ln_jitter=ln_jitter), np.float64)


# ------------------------------------------------------------------ elementary ops

def test_layer_norm_matches_library():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 7, 48)) * 3 + 1
    g, b = rng.standard_normal(48), rng.standard_normal(48)
    ref = F.layer_norm(torch.tensor(x), (48,), torch.tensor(g), torch.tensor(b), 1e-5).numpy()
    np.testing.assert_allclose(om.layer_norm(x, g, b, 1e-5), ref, rtol=0, atol=1e-12)
    # closed form: unit gain / zero bias -> zero mean, variance 1/(1 + eps/var)
    y = om.layer_norm(x, np.ones(48), np.zeros(48), 1e-5)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-12)
    var = x.var(-1)
    np.testing.assert_allclose(y.var(-1), var / (var + 1e-5), rtol=1e-12)


def test_gelu_closed_form_values():
    # x * Phi(x), Phi the standard normal CDF: Phi(1) = 0.8413447460685429
    xs = np.array([0.0, 1.0, -1.0, 2.0, -3.0])
    phi = np.array([0.5, 0.8413447460685429, 0.15865525393145707, 0.9772498680518208,
                    0.0013498980316301035])
    np.testing.assert_allclose(om.gelu(xs), xs * phi, rtol=1e-14, atol=1e-16)
    x = np.linspace(-6, 6, 1001)
    ref = F.gelu(torch.tensor(x), approximate="none").numpy()
    np.testing.assert_allclose(om.gelu(x), ref, rtol=1e-13, atol=1e-15)
    # the tanh approximation differs by more than rounding: the oracle is the exact form
    approx = F.gelu(torch.tensor(x), approximate="tanh").numpy()
    assert np.abs(om.gelu(x) - approx).max() > 1e-5


def test_rope_hand_example_and_pairing():
    # d = 4, base 100: frequencies 100^0 = 1 and 100^(-1/2) = 0.1; pairs (0,2) and (1,3)
    x = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 1, 4)
    y = om.apply_rope(x, np.array([2]), 100.0).ravel()
    a0, a1 = 2 * 1.0, 2 * 0.1
    expect = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
              3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    np.testing.assert_allclose(y, expect, rtol=1e-14)
    # position 0 is the identity
    np.testing.assert_array_equal(om.apply_rope(x, np.array([0]), 100.0), x)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 1, 64))
    k = rng.standard_normal((1, 1, 1, 64))
    for p in [0, 3, 77, 8191]:
        rq = om.apply_rope(q, np.array([p]), 1e4)
        assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) < 1e-12
    dots = []
    for shift in [0, 5, 1000]:
        rq = om.apply_rope(q, np.array([17 + shift]), 1e4)
        rk = om.apply_rope(k, np.array([9 + shift]), 1e4)
        dots.append(float((rq * rk).sum()))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 6, 3, 32))
    pos = np.arange(6) * 7
    ref = tc.rope_complex(torch.tensor(x).transpose(1, 2), torch.tensor(pos), 1e4).transpose(1, 2).numpy()
    np.testing.assert_allclose(om.apply_rope(x, pos, 1e4), ref, atol=1e-12)


def test_causal_attention_matches_library():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((2, 9, 3, 16)) for _ in range(3))
    pos = np.arange(9)
    out = om.causal_attention(q, k, v, pos, pos)
    t = lambda a: torch.tensor(a).transpose(1, 2)  # noqa: E731
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True).transpose(1, 2).numpy()
    np.testing.assert_allclose(out, ref, atol=1e-12)
    # one decode query at the last position == last row of the full causal result
    last = om.causal_attention(q[:, -1:], k, v, pos[-1:], pos)
    np.testing.assert_allclose(last[:, 0], out[:, -1], atol=1e-14)
    # brute force for one (b, h, i)
    b, h, i = 1, 2, 5
    s = np.array([q[b, i, h] @ k[b, j, h] / 4.0 for j in range(i + 1)])
    p = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    np.testing.assert_allclose(out[b, i, h], sum(p[j] * v[b, j, h] for j in range(i + 1)), atol=1e-14)


# ------------------------------------------------------------------ components

def test_embedder_brute_force():
    cfg = tiny()
    W = w64(cfg)
    rng = np.random.default_rng(5)
    x = rng.integers(0, cfg.vocab, (3, 12))
    e = om.embed_blocks(W, cfg, x)
    De = cfg.d_model // cfg.block_len
    assert e.shape == (3, 3, cfg.d_model)
    for b in range(3):
        for i in range(3):
            for o in range(cfg.block_len):
                for d in range(De):
                    assert e[b, i, o * De + d] == W["emb_block"][x[b, i * cfg.block_len + o], d]


def test_prefix_projection_layout():
    cfg = tiny(prefix_len=3)
    W = w64(cfg)
    c = np.random.default_rng(6).standard_normal((2, cfg.d_model))
    pre = om.prefix_from_context(W, cfg, c)
    D = cfg.d_model
    for b in range(2):
        for j in range(3):
            for d in range(0, D, 7):
                u = sum(c[b, i] * W["prefix.w"][i, j * D + d] for i in range(D)) + W["prefix.b"][j * D + d]
                assert abs(pre[b, j, d] - u) < 1e-12


def test_left_padding():
    cfg = tiny()
    x = np.arange(1, 31).reshape(1, 30)
    px = om.pad_prompt(cfg, x)
    assert px.shape == (1, 32)
    assert list(px[0, :2]) == [cfg.pad_id] * 2 and list(px[0, 2:]) == list(range(1, 31))
    assert om.pad_prompt(cfg, np.array([[7, 8]])).tolist() == [[0, 0, 7, 8]]
    assert om.pad_prompt(cfg, np.arange(8).reshape(1, 8)).shape == (1, 8)


def test_greedy_ties_lowest_id():
    lg = np.array([[0.1, 0.5, 0.5, -1.0], [2.0, 2.0, 2.0, 2.0]])
    assert om.greedy(lg).tolist() == [1, 0]


# ------------------------------------------------------------------ whole model

@pytest.mark.parametrize("kw", [dict(), dict(block_len=2, prefix_len=2), dict(block_len=1, prefix_len=2),
                                dict(block_len=8, prefix_len=1, d_model=64)])
def test_matches_library_crosscheck(kw):
    """Oracle full recompute vs the torch-library formulation, block by block."""
    cfg = tiny(**kw)
    W = w64(cfg)
    L = cfg.block_len
    x = np.random.default_rng(7).integers(0, cfg.vocab, (2, 4 * L))
    for k in (1, 2, 3):
        ref = tc.block_logits(W, cfg, x, k)
        got = om.logits_at(W, cfg, x, [k * L + o for o in range(L)])
        np.testing.assert_allclose(got, ref, atol=1e-11, rtol=0)


@pytest.mark.parametrize("kw,T,G", [(dict(), 32, 16), (dict(), 30, 13), (dict(block_len=1, prefix_len=2), 9, 7),
                                    (dict(block_len=2, prefix_len=2), 11, 9), (dict(block_len=8, prefix_len=2), 19, 18)])
def test_incremental_equals_full_recompute(kw, T, G):
    """Prefill + decode steps with caches == teacher-forced full recompute (float64)."""
    cfg = tiny(**kw)
    W = w64(cfg)
    prompt = wl.make_prompt(cfg, batch=2, T=T)
    ids, lg, st = om.generate(W, cfg, prompt, G, keep_logits=True)
    seq = np.concatenate([om.pad_prompt(cfg, prompt), ids], axis=1)
    Tp = seq.shape[1] - G
    full = om.logits_at(W, cfg, seq, range(Tp, Tp + G))
    assert np.abs(full - lg).max() <= 1e-10
    np.testing.assert_array_equal(om.greedy(full), ids)


def test_causality_bitwise():
    """Perturbing tokens at positions >= s leaves the logits of positions t <= s bit-identical."""
    cfg = tiny()
    W = w64(cfg)
    x = np.random.default_rng(8).integers(0, cfg.vocab, (2, 24))
    for s in (9, 12, 14):
        y = x.copy()
        y[:, s:] = (y[:, s:] + 101) % cfg.vocab
        a = om.logits_at(W, cfg, x, range(4, 25))
        b = om.logits_at(W, cfg, y, range(4, 25))
        t = np.arange(4, 25)
        np.testing.assert_array_equal(a[:, t <= s], b[:, t <= s])
        assert np.abs(a[:, t > s] - b[:, t > s]).max() > 1e-6


def test_token_decoder_locality():
    """Block k's logits are a function of c_{k-1} and block k's own tokens only."""
    cfg = tiny()
    W = w64(cfg)
    L, P = cfg.block_len, cfg.prefix_len
    x = np.random.default_rng(9).integers(0, cfg.vocab, (2, 20))
    k = 3
    c = om.context_embeddings(W, cfg, x, k)[:, k - 1]
    z = np.concatenate([om.prefix_from_context(W, cfg, c), W["emb_token"][x[:, k * L: k * L + L - 1]]], 1)
    local = om.output_logits(W, om.token_decoder(W, cfg, z)[:, P - 1:])
    full = om.logits_at(W, cfg, x, range(k * L, k * L + L))
    np.testing.assert_allclose(local, full, atol=1e-13)
    # changing an earlier block changes c_{k-1}, hence block k's logits (not vacuous)
    y = x.copy()
    y[:, 1] = (y[:, 1] + 5) % cfg.vocab
    assert np.abs(om.logits_at(W, cfg, y, range(k * L, k * L + L)) - full).max() > 1e-6


def test_kv_cache_lengths():
    """Block KV grows one entry per L_B tokens; the local KV is bounded and reset per block."""
    for kw, T in [(dict(), 32), (dict(block_len=2, prefix_len=2), 10), (dict(block_len=1, prefix_len=2), 7)]:
        cfg = tiny(**kw)
        W = w64(cfg, ln_jitter=False)
        L, P = cfg.block_len, cfg.prefix_len
        prompt = wl.make_prompt(cfg, batch=1, T=T)
        st, lg = om.prefill(W, cfg, prompt)
        Tp = wl.padded_len(cfg, T)
        ids = [om.greedy(lg)]
        for g in range(1, 14):
            assert st.block_kv_len == Tp // L + (g - 1) // L
            assert st.local_kv_len == P + (g - 1) % L <= P + L - 1
            ids.append(om.greedy(om.decode_step(W, cfg, st, ids[-1])))
        # a vanilla KV would hold every token: L_B times more entries
        assert (Tp + 13) // L == st.block_kv_len or L == 1


def test_golden_cost_model_numbers():
    """The reductions the pages print, reproduced by counting the oracle's KV reads."""
    gold = json.load(open(os.path.join(GOLDEN, "cost_model.json")))
    g = gold["block_decoder_input"]
    cfg = tiny(block_len=g["block_len"])
    assert om.pad_prompt(cfg, np.zeros((1, g["tokens"]), np.int64)).shape[1] // cfg.block_len == g["block_embeddings"]
    r = gold["token_decoder_kv_reduction"]
    assert r["context_len"] // r["block_len"] == r["R"]
    # block-decoder KV reads over a whole decode, vs a vanilla decoder's sum_{t<=Lseq} t
    f = gold["block_decoder_kv_io_reduction"]
    cfg = tiny(block_len=f["block_len"], d_model=64, n_block_layers=1, n_token_layers=1)
    W = w64(cfg, ln_jitter=False)
    G = 400
    _, _, st = om.generate(W, cfg, wl.make_prompt(cfg, batch=1, T=4), G)
    Lseq = 4 + G
    vanilla = Lseq * (Lseq + 1) // 2
    ratio = vanilla / st.kv_reads_block
    assert abs(ratio - f["factor"]) / f["factor"] < 0.05
    lb = gold["local_kv_bound"]
    cfg = tiny(block_len=lb["block_len"], prefix_len=lb["prefix_len"])
    W = w64(cfg, ln_jitter=False)
    st, lg = om.prefill(W, cfg, wl.make_prompt(cfg, batch=1, T=8))
    prev = om.greedy(lg)
    for _ in range(12):
        before = st.kv_reads_local
        prev = om.greedy(om.decode_step(W, cfg, st, prev))
        assert st.kv_reads_local - before <= lb["max_entries"]
        assert st.local_kv_len <= lb["max_entries"]


def test_float32_oracle_stays_float32():
    """The large-shape oracle runs in the dtype of its weights (no silent promotion to float64)."""
    cfg = tiny()
    W = om.weights_as(wl.make_weights(cfg), np.float32)
    ids, lg, st = om.generate(W, cfg, wl.make_prompt(cfg, batch=1, T=8), 6, keep_logits=True)
    assert lg.dtype == np.float32 and st.block_caches[0].k.dtype == np.float32
    assert om.gelu(np.ones(3, np.float32)).dtype == np.float32


@pytest.mark.parametrize("kv", [1, 2])
def test_grouped_query_attention_matches_library_and_incremental(kv):
    """n_kv_heads < n_heads: query head i attends with key/value head i // (H / n_kv_heads) (torch's
    grouped-query option of scaled_dot_product_attention); n_kv_heads = 1 is multi-query attention.
    Also pinned: the caches hold n_kv_heads heads, and the incremental path equals full recompute."""
    cfg = tiny(n_heads=4, n_kv_heads=kv, d_model=64)
    W = w64(cfg)
    assert W["blk.0.attn.qkv.w"].shape == (64, 64 + 2 * kv * 16)
    x = np.random.default_rng(12).integers(0, cfg.vocab, (2, 4 * cfg.block_len))
    for k in (1, 2, 3):
        np.testing.assert_allclose(om.logits_at(W, cfg, x, range(k * cfg.block_len, (k + 1) * cfg.block_len)),
                                   tc.block_logits(W, cfg, x, k), atol=1e-11)
    prompt = wl.make_prompt(cfg, batch=2, T=9)
    ids, lg, st = om.generate(W, cfg, prompt, 9, keep_logits=True)
    Tp = wl.padded_len(cfg, 9)
    seq = np.concatenate([om.pad_prompt(cfg, prompt), ids], axis=1)
    full = om.logits_at(W, cfg, seq, range(Tp, Tp + 9))
    assert np.abs(full - lg).max() <= 1e-10
    assert st.block_caches[0].k.shape[2] == kv and st.local_caches[0].k.shape[2] == kv


def test_grouped_query_with_full_groups_is_multi_head():
    """n_kv_heads = n_heads is ordinary multi-head attention: same weights, same logits."""
    cfg = tiny()
    W = w64(cfg)
    x = np.random.default_rng(13).integers(0, cfg.vocab, (2, 3 * cfg.block_len))
    a = om.logits_at(W, cfg, x, range(cfg.block_len, 3 * cfg.block_len))
    b = om.logits_at(W, cfg.with_(n_kv_heads=cfg.n_heads), x, range(cfg.block_len, 3 * cfg.block_len))
    assert np.array_equal(a, b)


def test_vanilla_mode_matches_library_and_incremental():
    """n_token_layers = 0, L_B = 1: a standard token-level decoder (the pages' Pythia baselines)."""
    cfg = tiny(n_token_layers=0, block_len=1, n_block_layers=3)
    W = w64(cfg)
    assert "emb_token" not in W and "prefix.w" not in W
    x = np.random.default_rng(11).integers(0, cfg.vocab, (2, 12))
    for t in (1, 5, 12):
        np.testing.assert_allclose(om.logits_at(W, cfg, x, [t])[:, 0], tc.vanilla_logits(W, cfg, x, t), atol=1e-11)
    prompt = wl.make_prompt(cfg, batch=2, T=7)
    ids, lg, st = om.generate(W, cfg, prompt, 9, keep_logits=True)
    seq = np.concatenate([prompt.astype(np.int64), ids], axis=1)
    full = om.logits_at(W, cfg, seq, range(7, 16))
    assert np.abs(full - lg).max() <= 1e-10
    assert st.block_kv_len == 7 + 8 and st.local_kv_len == 0


# ------------------------------------------------------------------ context injection variants
# §3.4 "The Token Decoder" compares prefix tokens with two alternatives: summation (MEGABYTE) and
# cross-attention.  Both run a local sequence led by one start slot (the pad token's embedding).

CONTEXT_VARIANTS = [dict(context_mode="sum"), dict(context_mode="sum", block_len=2),
                    dict(context_mode="xattn", prefix_len=2),
                    dict(context_mode="xattn", prefix_len=3, n_heads=4, n_kv_heads=2)]


@pytest.mark.parametrize("kw", CONTEXT_VARIANTS)
def test_context_variants_match_library_crosscheck(kw):
    """Summation and cross-attention injection vs the torch-library formulation, block by block."""
    cfg = tiny(**kw)
    W = w64(cfg)
    L = cfg.block_len
    x = np.random.default_rng(21).integers(0, cfg.vocab, (2, 4 * L))
    for k in (1, 2, 3):
        np.testing.assert_allclose(om.logits_at(W, cfg, x, [k * L + o for o in range(L)]),
                                   tc.block_logits(W, cfg, x, k), atol=1e-11, rtol=0)


@pytest.mark.parametrize("kw", CONTEXT_VARIANTS)
def test_context_variants_incremental_and_causal(kw):
    """Incremental decoding == full recompute; the local cache holds the start slot plus the
    block's tokens; perturbing later tokens leaves earlier logits bit-identical."""
    cfg = tiny(**kw)
    W = w64(cfg)
    prompt = wl.make_prompt(cfg, batch=2, T=11)
    G = 10
    ids, lg, st = om.generate(W, cfg, prompt, G, keep_logits=True)
    seq = np.concatenate([om.pad_prompt(cfg, prompt), ids], axis=1)
    Tp = seq.shape[1] - G
    full = om.logits_at(W, cfg, seq, range(Tp, Tp + G))
    assert np.abs(full - lg).max() <= 1e-10
    assert cfg.lead == 1 and st.local_kv_len == 1 + (G - 1) % cfg.block_len
    x = np.random.default_rng(22).integers(0, cfg.vocab, (2, 24))
    s = 13
    y = x.copy()
    y[:, s:] = (y[:, s:] + 57) % cfg.vocab
    t = np.arange(cfg.block_len, 25)
    a, b = om.logits_at(W, cfg, x, t), om.logits_at(W, cfg, y, t)
    np.testing.assert_array_equal(a[:, t <= s], b[:, t <= s])
    assert np.abs(a[:, t > s] - b[:, t > s]).max() > 1e-6


def test_summation_with_one_token_blocks_is_one_prefix_vector():
    """With L_B = 1 the summation design has one local slot, start + u_0; with a zero pad-token
    embedding that is u_0 = Proj(c), the single prefix vector of the P = 1 prefix design."""
    cfg_p = tiny(block_len=1, prefix_len=1)
    cfg_s = cfg_p.with_(context_mode="sum")
    W = w64(cfg_p)
    assert [s for s in wl.weight_specs(cfg_p)] == [s for s in wl.weight_specs(cfg_s)]
    x = np.random.default_rng(23).integers(1, cfg_p.vocab, (2, 8))
    t = range(1, 9)
    assert np.abs(om.logits_at(W, cfg_p, x, t) - om.logits_at(W, cfg_s, x, t)).max() > 1e-6
    W["emb_token"][cfg_p.pad_id] = 0.0
    np.testing.assert_array_equal(om.logits_at(W, cfg_p, x, t), om.logits_at(W, cfg_s, x, t))


def test_cross_attention_over_one_state_ignores_the_query():
    """With P = 1 the cross-attention softmax has a single term of weight exactly 1, so the branch
    adds the projected value whatever the queries: new query weights leave the logits bit-identical,
    new value biases do not."""
    cfg = tiny(context_mode="xattn", prefix_len=1)
    W = w64(cfg)
    rng = np.random.default_rng(24)
    x = rng.integers(0, cfg.vocab, (2, 16))
    t = range(4, 17)
    ref = om.logits_at(W, cfg, x, t)
    Wq, Wv = dict(W), dict(W)
    kvw = cfg.kv_heads * cfg.d_head
    for l in range(cfg.n_token_layers):
        Wq[f"tok.{l}.xattn.q.w"] = rng.standard_normal(W[f"tok.{l}.xattn.q.w"].shape)
        Wq[f"tok.{l}.xattn.q.b"] = rng.standard_normal(W[f"tok.{l}.xattn.q.b"].shape)
        Wv[f"tok.{l}.xattn.kv.b"] = W[f"tok.{l}.xattn.kv.b"] + np.r_[np.zeros(kvw), np.full(kvw, 0.5)]
    np.testing.assert_array_equal(om.logits_at(Wq, cfg, x, t), ref)
    assert np.abs(om.logits_at(Wv, cfg, x, t) - ref).max() > 1e-6


def test_cross_attention_with_equal_scores_averages_the_values():
    """A zero query projection gives every encoder state the same score, so the cross-attention
    branch of a layer is the mean of the P projected values through the output projection."""
    cfg = tiny(context_mode="xattn", prefix_len=3)
    W = w64(cfg)
    rng = np.random.default_rng(25)
    name, D = "tok.0", cfg.d_model
    W[f"{name}.xattn.q.w"] = np.zeros_like(W[f"{name}.xattn.q.w"])
    W[f"{name}.xattn.q.b"] = np.zeros_like(W[f"{name}.xattn.q.b"])
    h = rng.standard_normal((2, 5, D))
    enc = rng.standard_normal((2, 3, D))
    pos = np.arange(5)
    args = (W, name, h, pos, cfg.n_heads, cfg.ln_eps, cfg.rope_base)
    branch = om.layer_forward(*args, None, 0, enc) - om.layer_forward(*args)
    v = enc @ W[f"{name}.xattn.kv.w"][:, D:] + W[f"{name}.xattn.kv.b"][D:]     # [2, P, D] values
    want = v.mean(axis=1) @ W[f"{name}.xattn.out.w"] + W[f"{name}.xattn.out.b"]
    np.testing.assert_allclose(branch, np.broadcast_to(want[:, None], branch.shape), atol=1e-12, rtol=0)
