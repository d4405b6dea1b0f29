"""End-to-end parity of the HIP path with the oracle on small models, every generation step:
fp32 (1e-4 max-abs logits, greedy ids identical) and bf16 (2e-2, ids within the tolerance band),
plus the cache contents, cache lengths, determinism and host-side error paths."""
import ctypes

import numpy as np
import pytest

import bt_workloads as wl
from oracle import model as om
from tests.gpu_harness import (BF16_TOL, FP32_TOL, check_ids_against, log, require_gpu, run_gpu,
                               teacher_forced_logits)

pytestmark = pytest.mark.gpu

SMALL_BF16 = wl.Config("small_bf16", "bf16", vocab=512, d_model=128, n_heads=2, d_mlp=512, n_block_layers=2,
                       n_token_layers=2, block_len=4, prefix_len=2, batch=5, prompt_len=37, gen_len=20)


def _fp32_case(cfg, B, T, G, seed=0):
    log(f"fp32 case {cfg.name} L_B={cfg.block_len} P={cfg.prefix_len} B={B} T={T} G={G}")
    W = wl.make_weights(cfg, seed=seed, ln_jitter=True)
    prompt = wl.make_prompt(cfg, batch=B, T=T, seed=seed)
    ids, lg, model = run_gpu(cfg, W, prompt, G, logits_steps=range(G))
    W64 = om.weights_as(W, np.float64)
    ref_ids, ref_lg, st = om.generate(W64, cfg, prompt, G, keep_logits=True)
    gl = np.stack([lg[g] for g in range(G)], axis=1)
    err = np.abs(gl - ref_lg).max()
    log(f"  max-abs logit error {err:.3e}")
    assert err <= FP32_TOL
    np.testing.assert_array_equal(ids, ref_ids)
    assert model.cache_lengths() == (st.block_kv_len, st.local_kv_len)
    return model


def test_c0_tiny_fp32_full():
    cfg = wl.get_config("c0_tiny")
    _fp32_case(cfg, cfg.batch, cfg.prompt_len, cfg.gen_len)


@pytest.mark.parametrize("kw,B,T,G", [(dict(), 3, 30, 13), (dict(block_len=1, prefix_len=2), 2, 9, 7),
                                      (dict(block_len=2, prefix_len=2), 3, 11, 10),
                                      (dict(block_len=8, prefix_len=2), 2, 19, 18),
                                      (dict(d_model=128, n_heads=2), 2, 8, 9),
                                      (dict(d_model=256, n_heads=2, d_mlp=320), 2, 12, 6),
                                      # degenerate sizes: one row, a one-token prompt (one block, all
                                      # but its last slot padding), no decode step or a few
                                      (dict(), 1, 1, 1), (dict(), 1, 1, 9),
                                      (dict(block_len=8, prefix_len=2), 1, 1, 3)])
def test_fp32_variants(kw, B, T, G):
    _fp32_case(wl.get_config("c0_tiny", **kw), B, T, G, seed=1)


# grouped-query attention: groups of 2 (one decode workgroup per KV head), 3 (a workgroup with an
# idle head slot), 8 (a group cut into two runs of 4) and multi-query with L_B = 2
GQA_FP32 = [(dict(d_model=128, n_heads=4, n_kv_heads=2), 2, 10, 9),
            (dict(d_model=192, n_heads=6, n_kv_heads=2, d_mlp=320), 3, 13, 8),
            (dict(d_model=256, n_heads=8, n_kv_heads=1), 2, 9, 7),
            (dict(d_model=128, n_heads=4, n_kv_heads=1, block_len=2, prefix_len=2), 2, 11, 10)]


@pytest.mark.parametrize("kw,B,T,G", GQA_FP32)
def test_fp32_grouped_query_attention(kw, B, T, G):
    _fp32_case(wl.get_config("c0_tiny", **kw), B, T, G, seed=13)


# context injection by summation (L_B summands; L_B = 1 is a single slot) and by cross-attention
# (P encoder states; P = 1 is a single state), with grouped-query heads in one case
CONTEXT_FP32 = [(dict(context_mode="sum"), 3, 13, 11), (dict(context_mode="sum", block_len=2), 2, 9, 8),
                (dict(context_mode="sum", block_len=1), 2, 7, 6),
                (dict(context_mode="xattn", prefix_len=2), 3, 13, 11),
                (dict(context_mode="xattn", prefix_len=1, block_len=2), 2, 9, 8),
                (dict(context_mode="xattn", prefix_len=3, d_model=128, n_heads=4, n_kv_heads=2), 2, 10, 9)]


@pytest.mark.parametrize("kw,B,T,G", CONTEXT_FP32)
def test_fp32_context_injection_variants(kw, B, T, G):
    _fp32_case(wl.get_config("c0_tiny", **kw), B, T, G, seed=16)


@pytest.mark.parametrize("kw", [dict(context_mode="sum"), dict(context_mode="xattn", prefix_len=3),
                                dict(context_mode="xattn", prefix_len=2, d_model=512, n_heads=4, n_kv_heads=2),
                                dict(context_mode="sum", block_len=8)])
def test_bf16_context_injection_variants(kw):
    """bf16 every step for both variants (d_head 64, and 128 with grouped-query heads)."""
    cfg = SMALL_BF16.with_(**kw)
    log(f"bf16 context-variant case {kw}")
    W = wl.make_weights(cfg, seed=17, ln_jitter=True)
    prompt = wl.make_prompt(cfg, seed=17)
    G = cfg.gen_len
    ids, lg, model = run_gpu(cfg, W, prompt, G, logits_steps=range(G))
    _, ref_lg, st = om.generate(om.weights_as(W, np.float64), cfg, prompt, G, keep_logits=True, forced=ids)
    gl = np.stack([lg[g] for g in range(G)], axis=1)
    err = np.abs(gl - ref_lg).max()
    exact = check_ids_against(ref_lg, ids, BF16_TOL)
    log(f"  max-abs logit error {err:.3e}, exact argmax {exact:.3f}")
    assert err <= BF16_TOL
    assert model.cache_lengths() == (st.block_kv_len, st.local_kv_len)


@pytest.mark.parametrize("kw,max_tokens", [(dict(d_model=256, n_heads=4, n_kv_heads=2), None),
                                           (dict(d_model=384, n_heads=6, n_kv_heads=2, d_mlp=768), None),
                                           (dict(d_model=256, n_heads=4, n_kv_heads=1), 4096),
                                           (dict(d_model=512, n_heads=4, n_kv_heads=2), None)])
def test_bf16_grouped_query_attention(kw, max_tokens):
    """bf16 GQA / MQA every step; max_tokens=4096 adds key splits, d_model=512 gives d_head=128."""
    cfg = SMALL_BF16.with_(**kw)
    log(f"bf16 GQA case {kw} max_tokens={max_tokens}")
    W = wl.make_weights(cfg, seed=14, ln_jitter=True)
    prompt = wl.make_prompt(cfg, seed=14)
    G = cfg.gen_len
    ids, lg, model = run_gpu(cfg, W, prompt, G, logits_steps=range(G), max_tokens=max_tokens)
    _, ref_lg, st = om.generate(om.weights_as(W, np.float64), cfg, prompt, G, keep_logits=True, forced=ids)
    gl = np.stack([lg[g] for g in range(G)], axis=1)
    err = np.abs(gl - ref_lg).max()
    exact = check_ids_against(ref_lg, ids, BF16_TOL)
    log(f"  max-abs logit error {err:.3e}, exact argmax {exact:.3f}")
    assert err <= BF16_TOL
    assert model.cache_lengths() == (st.block_kv_len, st.local_kv_len)


@pytest.mark.parametrize("kw,max_tokens", [(dict(), None), (dict(d_model=256, n_heads=2), None),
                                           (dict(block_len=1, prefix_len=1), None), (dict(block_len=8, prefix_len=2), None),
                                           (dict(), 4096), (dict(batch=1, prompt_len=1, gen_len=9), None)])
def test_bf16_small_every_step(kw, max_tokens):
    """max_tokens=4096 gives the block attention several key splits, most of them still empty."""
    cfg = SMALL_BF16.with_(**kw)
    log(f"bf16 case {kw} max_tokens={max_tokens}")
    W = wl.make_weights(cfg, seed=2, ln_jitter=True)
    prompt = wl.make_prompt(cfg, seed=2)
    G = cfg.gen_len
    ids, lg, model = run_gpu(cfg, W, prompt, G, logits_steps=range(G), max_tokens=max_tokens)
    W64 = om.weights_as(W, np.float64)
    _, ref_lg, st = om.generate(W64, cfg, prompt, G, keep_logits=True, forced=ids)
    gl = np.stack([lg[g] for g in range(G)], axis=1)
    err = np.abs(gl - ref_lg).max()
    exact = check_ids_against(ref_lg, ids, BF16_TOL)
    log(f"  max-abs logit error {err:.3e}, exact argmax {exact:.3f}")
    assert err <= BF16_TOL
    assert model.cache_lengths() == (st.block_kv_len, st.local_kv_len)


@pytest.mark.parametrize("kw,B", [(dict(), 1), (dict(), 5), (dict(d_model=256, n_heads=4), 40),
                                  (dict(d_model=256, n_heads=4, n_kv_heads=2), 100),
                                  (dict(d_model=384, n_heads=6, n_kv_heads=1, d_mlp=768), 200),
                                  (dict(context_mode="sum"), 70), (dict(block_len=8, prefix_len=3), 130),
                                  (dict(context_mode="xattn", prefix_len=2), 70),
                                  (dict(context_mode="xattn", prefix_len=3, d_model=256, n_heads=4, n_kv_heads=2), 130),
                                  (dict(d_model=256, n_heads=4, d_mlp=1536), 256),
                                  (dict(context_mode="xattn", prefix_len=2, d_model=256, n_heads=4, d_mlp=1536), 256)])
def test_fused_local_attention_out_gemm(kw, B):
    """The token decoder's local attention (and, with cross-attention injection, the
    cross-attention over the P encoder states) computed inside its [out|down] GEMM (the default
    decode path for fp16 with head width 64) against the oracle at every step, and against the
    separate launches. Batches of 1 to 256 rows cover every workgroup shape of the fused kernel
    (16, 32, 64 and 128 rows per workgroup up to 128 rows; above that, 64-row workgroups over row
    groups), one to eight 32-row attention blocks, and one, two and several K splits of the GELU
    columns (256 rows with a 1536-wide MLP: two splits, the largest batch the fused launch takes).
    Local windows up to 11 entries take the loop over cached keys past its first group of four."""
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    cfg = SMALL_BF16.with_(batch=B, **kw)
    log(f"fused local attention case {kw} B={B}")
    W = wl.make_weights(cfg, seed=21, ln_jitter=True)
    prompt = wl.make_prompt(cfg, seed=21)
    G = cfg.gen_len
    d_prompt = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    mt = wl.padded_len(cfg, prompt.shape[1]) + G
    runs = {}
    for fused in (True, False):
        model = hg.BlockTransformer(cfg, W, max_batch=B, max_tokens=mt)
        model.set_fuse_local(fused)
        ids, lg = model.generate(d_prompt, G, logits_steps=range(G))
        torch.cuda.synchronize()
        runs[fused] = (ids.cpu().numpy().T.copy(), np.stack([lg[g].cpu().numpy() for g in range(G)], axis=1))
        del model
    ids, gl = runs[True]
    _, ref_lg, _ = om.generate(om.weights_as(W, np.float64), cfg, prompt, G, keep_logits=True, forced=ids)
    err = np.abs(gl - ref_lg).max()
    exact = check_ids_against(ref_lg, ids, BF16_TOL)
    ids_s, gl_s = runs[False]
    same = ids == ids_s
    log(f"  fused: max-abs logit error {err:.3e}, exact argmax {exact:.3f}; ids equal to the separate "
        f"launches {same.mean():.3f}")
    assert err <= BF16_TOL
    # up to the first step where the two id streams part, the logits agree within the tolerance
    first = int(np.argmin(same.all(axis=0))) if not same.all() else G
    if first > 0:
        assert np.abs(gl[:, :first] - gl_s[:, :first]).max() <= BF16_TOL


@pytest.mark.parametrize("B", [65, 100, 128])
def test_wide_model_decode_gemms_65_to_128_rows(B):
    """Decode at 65-128 rows of a d = 2048 model: the [q|k|v|up] GEMM (8192 columns) and the
    [out|down] GEMM (K = 4096, 8 K splits folded by the next LayerNorm) run with one wave holding
    all rows over 64 columns.  Every step's logits against the oracle on the GPU's ids."""
    cfg = SMALL_BF16.with_(d_model=2048, n_heads=16, d_mlp=2048, batch=B, prompt_len=9, gen_len=7)
    log(f"wide decode case B={B}")
    W = wl.make_weights(cfg, seed=29, ln_jitter=True)
    prompt = wl.make_prompt(cfg, seed=29)
    G = cfg.gen_len
    ids, lg, model = run_gpu(cfg, W, prompt, G, logits_steps=range(G))
    model.close()
    del model
    _, ref_lg, _ = om.generate(om.weights_as(W, np.float64), cfg, prompt, G, keep_logits=True, forced=ids)
    gl = np.stack([lg[g] for g in range(G)], axis=1)
    err = np.abs(gl - ref_lg).max()
    exact = check_ids_against(ref_lg, ids, BF16_TOL)
    log(f"  max-abs logit error {err:.3e}, exact argmax {exact:.3f}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("D", [1024, 1536])
def test_wide_model_prefill_layernorm(D):
    """Prefill of more than 1024 block rows at widths above 768: the block decoder's LayerNorms run
    on the kernel that writes 16-byte operand pieces from registers (1024: two column octets a lane;
    1536: three of four, the last masked).  Every row's first token and two decode steps against
    the oracle."""
    cfg = SMALL_BF16.with_(d_model=D, n_heads=D // 128, d_mlp=512, prefix_len=1, batch=3, prompt_len=1399, gen_len=3)
    T = wl.padded_len(cfg, cfg.prompt_len)
    log(f"wide prefill case D={D}: {cfg.batch} x {T // cfg.block_len} block rows")
    assert cfg.batch * T // cfg.block_len > 1024
    W = wl.make_weights(cfg, seed=23, ln_jitter=True)
    prompt = wl.make_prompt(cfg, seed=23)
    G = cfg.gen_len
    ids, lg, model = run_gpu(cfg, W, prompt, G, logits_steps=range(G))
    model.close()
    del model
    worst = 0.0
    for r in range(cfg.batch):
        ref = teacher_forced_logits(cfg, W, prompt[r], ids[r], range(G))
        err = float(np.abs(np.stack([lg[g][r] for g in range(G)]) - ref).max())
        worst = max(worst, err)
        check_ids_against(ref, ids[r], BF16_TOL)
    log(f"  max-abs logit error {worst:.3e} over {cfg.batch} rows x {G} steps")
    assert worst <= BF16_TOL


@pytest.mark.parametrize("kw", [dict(), dict(d_model=256, n_heads=4, n_kv_heads=1)])
def test_deep_split_kv_long_context(kw):
    """12000 prompt blocks (L_B = 1) in the largest block-KV capacity, 131072 entries: the block
    attention runs its deepest split (32 splits of 4096 keys; 128 splits of 1024 keys when a
    workgroup serves a group of 4 query heads) and merges several non-empty splits every step."""
    cfg = SMALL_BF16.with_(block_len=1, prefix_len=2, **kw)
    B, T, G = 2, 12000, 5
    log(f"deep split-KV case {kw} B={B} T={T} G={G}")
    W = wl.make_weights(cfg, seed=15, ln_jitter=True)
    prompt = wl.make_prompt(cfg, batch=B, T=T, seed=15)
    ids, lg, model = run_gpu(cfg, W, prompt, G, logits_steps=range(G), max_tokens=131072)
    assert model.cache_lengths()[0] == T + G - 1
    model.close()
    del model
    for r in range(B):
        ref = teacher_forced_logits(cfg, W, prompt[r], ids[r], range(G))
        err = float(np.abs(np.stack([lg[g][r] for g in range(G)]) - ref).max())
        log(f"  row {r}: max-abs logit error {err:.3e}")
        assert err <= BF16_TOL
        check_ids_against(ref, ids[r], BF16_TOL)


@pytest.mark.parametrize("kw", [dict(), dict(d_model=256, n_heads=2)])
def test_block_attention_one_wave_per_unit(kw):
    """1024 rows x 2 heads = 2048 (row, head) units: the multi-head block attention runs one wave
    per unit (with fewer units four waves share one); head widths 64 and 128.  Rows 0, 511 and 1023
    are teacher-forced through the oracle at every step."""
    cfg = SMALL_BF16.with_(**kw)
    B, T, G = 1024, 37, 12
    log(f"one-wave block attention case {kw} B={B} T={T} G={G}")
    W = wl.make_weights(cfg, seed=16, ln_jitter=True)
    prompt = wl.make_prompt(cfg, batch=B, T=T, seed=16)
    ids, lg, model = run_gpu(cfg, W, prompt, G, logits_steps=range(G))
    model.close()
    del model
    for r in (0, 511, B - 1):
        ref = teacher_forced_logits(cfg, W, prompt[r], ids[r], range(G))
        err = float(np.abs(np.stack([lg[g][r] for g in range(G)]) - ref).max())
        log(f"  row {r}: max-abs logit error {err:.3e}")
        assert err <= BF16_TOL
        check_ids_against(ref, ids[r], BF16_TOL)


@pytest.mark.parametrize("kw", [dict(), dict(d_model=256, n_heads=4, n_kv_heads=2)])
def test_kv_caches_hold_rotated_keys_and_values(kw):
    """Block-KV (keys [slot][d], values in transposed groups of 8 slots [slot / 8][d][8]) and
    local-KV contents equal the oracle's caches (H_kv heads per row under grouped-query attention)."""
    torch = require_gpu()
    cfg = SMALL_BF16.with_(**kw)
    W = wl.make_weights(cfg, seed=3, ln_jitter=True)
    prompt = wl.make_prompt(cfg, seed=3)
    G = 7   # ends inside a block: local KV holds P + 2 entries
    ids, _, model = run_gpu(cfg, W, prompt, G, max_tokens=64)
    _, _, st = om.generate(om.weights_as(W, np.float64), cfg, prompt, G, forced=ids)
    B, H, dh = prompt.shape[0], cfg.kv_heads, cfg.d_head
    blk, cap = model.cache_view(0)
    blk = blk.cpu().float().numpy().reshape(cfg.n_block_layers, 2, B, H, cap, dh)
    n = st.block_kv_len
    for l in range(cfg.n_block_layers):
        k_ref = st.block_caches[l].k.transpose(0, 2, 1, 3)            # [B, H, n, dh]
        v_ref = st.block_caches[l].v.transpose(0, 2, 3, 1)            # [B, H, dh, n]
        k_gpu = blk[l, 0, :, :, :n, :]
        v_gpu = blk[l, 1].reshape(B, H, cap // 8, dh, 8).transpose(0, 1, 3, 2, 4).reshape(B, H, dh, cap)[:, :, :, :n]
        assert np.abs(k_gpu - k_ref).max() <= 2e-2 * max(1.0, np.abs(k_ref).max())
        assert np.abs(v_gpu - v_ref).max() <= 2e-2 * max(1.0, np.abs(v_ref).max())
    loc, lcap = model.cache_view(1)
    loc = loc.cpu().float().numpy().reshape(cfg.n_token_layers, 2, B, H, lcap, dh)
    m = st.local_kv_len
    for l in range(cfg.n_token_layers):
        k_ref = st.local_caches[l].k.transpose(0, 2, 1, 3)
        v_ref = st.local_caches[l].v.transpose(0, 2, 1, 3)
        assert np.abs(loc[l, 0, :, :, :m] - k_ref).max() <= 2e-2 * max(1.0, np.abs(k_ref).max())
        assert np.abs(loc[l, 1, :, :, :m] - v_ref).max() <= 2e-2 * max(1.0, np.abs(v_ref).max())


def test_cache_lengths_and_ratio():
    """Block KV grows one entry per L_B tokens (L_B times shorter than a token-level cache);
    local KV stays within P + L_B - 1 and restarts at P every block."""
    require_gpu()
    for L in (1, 2, 4):
        cfg = SMALL_BF16.with_(block_len=L, prefix_len=2)
        W = wl.make_weights(cfg, seed=4)
        prompt = wl.make_prompt(cfg, batch=2, T=16, seed=4)
        import torch
        import hierarchical_global_local_amd as hg
        model = hg.BlockTransformer(cfg, W, max_batch=2, max_tokens=64)
        d_prompt = torch.from_numpy(prompt).cuda()
        model.prefill(d_prompt)
        Tp = wl.padded_len(cfg, 16)
        for g in range(1, 30):
            assert model.cache_lengths() == (Tp // L + (g - 1) // L, 2 + (g - 1) % L)
            model.decode_step()
        torch.cuda.synchronize()


def test_deterministic_runs():
    cfg = SMALL_BF16
    W = wl.make_weights(cfg, seed=5)
    prompt = wl.make_prompt(cfg, seed=5)
    a = run_gpu(cfg, W, prompt, 12, logits_steps=[0, 5, 11])
    b = run_gpu(cfg, W, prompt, 12, logits_steps=[0, 5, 11])
    np.testing.assert_array_equal(a[0], b[0])
    for g in (0, 5, 11):
        np.testing.assert_array_equal(a[1][g], b[1][g])


def test_host_side_errors():
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    cfg = SMALL_BF16
    W = wl.make_weights(cfg, seed=6)
    model = hg.BlockTransformer(cfg, W, max_batch=2, max_tokens=16)
    with pytest.raises(hg.BtError) as e:
        model.decode_step(out=torch.empty(2, dtype=torch.int32, device="cuda"))
    assert e.value.code == -3
    with pytest.raises(hg.BtError) as e:
        model.prefill(torch.zeros((3, 8), dtype=torch.int32, device="cuda"))
    assert e.value.code == -2
    with pytest.raises(hg.BtError) as e:
        model.prefill(torch.zeros((1, 16), dtype=torch.int32, device="cuda"))
    assert e.value.code == -2
    # empty inputs: no rows, or rows without a token, are argument errors (nothing is queued)
    for shape in ((0, 8), (2, 0)):
        with pytest.raises(hg.BtError) as e:
            model.prefill(torch.zeros(shape, dtype=torch.int32, device="cuda"))
        assert e.value.code == -1
    with pytest.raises(hg.BtError) as e:
        model.decode_step(out=torch.empty(2, dtype=torch.int32, device="cuda"))
    assert e.value.code == -3   # still no prefill
    short = hg.BlockTransformer(cfg, W, max_batch=2, max_tokens=16, max_prompt_tokens=8)
    with pytest.raises(hg.BtError) as e:
        short.prefill(torch.zeros((2, 9), dtype=torch.int32, device="cuda"))   # padded to 12 > 8
    assert e.value.code == -2
    short.prefill(torch.zeros((2, 8), dtype=torch.int32, device="cuda"))
    model.prefill(torch.zeros((2, 11), dtype=torch.int32, device="cuda"))   # padded to 12, room for 4 tokens
    for _ in range(3):
        model.decode_step()
    with pytest.raises(hg.BtError) as e:
        model.decode_step()
    assert e.value.code == -2
    torch.cuda.synchronize()


@pytest.mark.parametrize("kw", [dict(), dict(block_len=1, prefix_len=2), dict(context_mode="sum"),
                                dict(context_mode="xattn", prefix_len=3)])
def test_graph_replay_matches_eager(kw):
    """Decode steps replayed from HIP graphs give the eagerly launched results bit for bit, over
    repeated replays with other GPU work and synchronisations in between, and when steps that ask
    for logits (launched eagerly) are interleaved with replayed ones."""
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    cfg = SMALL_BF16.with_(**kw)
    W = wl.make_weights(cfg, seed=7, ln_jitter=True)
    prompt = torch.from_numpy(wl.make_prompt(cfg, seed=7)).cuda()
    G = 23
    eager = hg.BlockTransformer(cfg, W, max_batch=5, max_tokens=128, graphs=False)
    ref_ids, ref_lg = eager.generate(prompt, G, logits_steps=range(G))
    torch.cuda.synchronize()
    graph = hg.BlockTransformer(cfg, W, max_batch=5, max_tokens=128, graphs=True)
    for rep in range(3):
        ids, lg = graph.generate(prompt, G, logits_steps=[3, 9] if rep == 1 else [])
        junk = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids), f"replay {rep}"
        for g, v in lg.items():
            assert torch.equal(v, ref_lg[g])
        del junk


def test_vanilla_mode_fp32_and_bf16_every_step():
    """n_token_layers = 0: a token-level transformer on the same kernels (the pages' baselines)."""
    cfg = wl.get_config("c0_tiny", n_token_layers=0, block_len=1, n_block_layers=3)
    _fp32_case(cfg, 2, 11, 9, seed=8)
    cfg = SMALL_BF16.with_(n_token_layers=0, block_len=1, n_block_layers=3)
    W = wl.make_weights(cfg, seed=8, ln_jitter=True)
    prompt = wl.make_prompt(cfg, seed=8)
    G = 15
    ids, lg, model = run_gpu(cfg, W, prompt, G, logits_steps=range(G))
    _, ref_lg, st = om.generate(om.weights_as(W, np.float64), cfg, prompt, G, keep_logits=True, forced=ids)
    gl = np.stack([lg[g] for g in range(G)], axis=1)
    assert np.abs(gl - ref_lg).max() <= BF16_TOL
    check_ids_against(ref_lg, ids, BF16_TOL)
    assert model.cache_lengths() == (st.block_kv_len, 0)


def test_kernel_replay_leaves_decoding_unchanged():
    """bt_test_replay (used by the benchmark to time one kernel class) may only overwrite
    activations, split-K partials and the not-yet-valid block-KV and local-KV slots: decoding
    after it is bit-identical."""
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    cfg = SMALL_BF16
    W = wl.make_weights(cfg, seed=11, ln_jitter=True)
    prompt = wl.make_prompt(cfg, seed=11)
    G = 14
    ref, _, _ = run_gpu(cfg, W, prompt, G)
    model = hg.BlockTransformer(cfg, W, max_batch=prompt.shape[0], max_tokens=wl.padded_len(cfg, prompt.shape[1]) + G)
    d_prompt = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    ids = torch.empty((G, prompt.shape[0]), dtype=torch.int32, device="cuda")
    with torch.cuda.stream(model.stream):
        model.prefill(d_prompt, ids[0])
        for g in range(1, G):
            if g in (3, 4, 7):  # after token steps and after a block step
                model.replay("gemm_qkv_up", 5)
                model.replay("local_attn_out", 5)
                model.replay("attn_block_decode", 5)
                model.replay("empty", 5)
            model.decode_step(ids[g])
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy().T, ref)
    with pytest.raises(hg.BtError):
        model.replay("layernorm", 1)


@pytest.mark.parametrize("name", ["c0_tiny", "small_bf16"])
def test_per_row_prompt_lengths(name):
    """bt_prefill_lengths: each row left-padded to the common length equals bt_prefill on the
    host-padded prompt (bit for bit) and the oracle on it (pad tokens are ordinary tokens)."""
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    cfg = SMALL_BF16 if name == "small_bf16" else wl.get_config("c0_tiny")
    W = wl.make_weights(cfg, seed=12, ln_jitter=True)
    B, T, G = 5, 23, 10
    rng = np.random.default_rng(12)
    lengths = np.array([23, 1, 9, 16, 4], dtype=np.int32)
    prompt = rng.integers(0, cfg.vocab, (B, T)).astype(np.int32)          # tokens past a row's length are junk
    Tp = wl.padded_len(cfg, T)
    padded = np.full((B, Tp), cfg.pad_id, dtype=np.int32)
    for b in range(B):
        padded[b, Tp - lengths[b]:] = prompt[b, :lengths[b]]
    ref_ids, ref_lg, _ = run_gpu(cfg, W, padded, G, logits_steps=range(G))
    model = hg.BlockTransformer(cfg, W, max_batch=B, max_tokens=Tp + G)
    ids = torch.empty((G, B), dtype=torch.int32, device="cuda")
    lg = torch.empty((G, B, cfg.vocab), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(model.stream):
        model.prefill(torch.from_numpy(prompt).cuda(), ids[0], lg[0], lengths=torch.from_numpy(lengths).cuda())
        for g in range(1, G):
            model.decode_step(ids[g], lg[g])
    torch.cuda.synchronize()
    got = ids.cpu().numpy().T
    assert np.array_equal(got, ref_ids)
    for g in range(G):
        np.testing.assert_array_equal(lg[g].cpu().numpy(), ref_lg[g])
    _, oracle_lg, _ = om.generate(om.weights_as(W, np.float64), cfg, padded, G, keep_logits=True, forced=got)
    tol = FP32_TOL if cfg.dtype == "fp32" else BF16_TOL
    assert np.abs(np.stack([lg[g].cpu().numpy() for g in range(G)], axis=1) - oracle_lg).max() <= tol
