"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every function the
headers declare, validates configs on the host and sizes the weights blob and workspace."""
import ctypes
import os
import re

import numpy as np
import pytest

import bt_workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in ("bt.h", "bt_test.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+(bt_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    import hierarchical_global_local_amd as hg
    L = hg.lib()
    names = declared_functions()
    assert {"bt_init", "bt_prefill", "bt_decode_step", "bt_destroy", "bt_weights_bytes"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def _cfg(name, **kw):
    import hierarchical_global_local_amd as hg
    c = wl.get_config(name, **kw)
    return c, hg.BtConfig.make(c, c.batch, wl.padded_len(c, c.prompt_len) + c.gen_len)


@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_blob_size_matches_packer(name):
    import hierarchical_global_local_amd as hg
    c, cfg = _cfg(name)
    n = sum(int(np.prod(s)) for _, s, _ in wl.weight_specs(c))
    elem = 4 if c.dtype == "fp32" else 2
    assert hg.lib().bt_weights_bytes(ctypes.byref(cfg)) == n * elem
    assert hg.weight_names(c) == [s[0] for s in wl.weight_specs(c)]


@pytest.mark.parametrize("kv", [1, 3, 4])
def test_grouped_query_blob_and_cache_sizes(kv):
    """With n_kv_heads the q|k|v projection is D + 2 H_kv d_head wide and both KV caches hold H_kv
    heads: H / H_kv times smaller than with multi-head attention."""
    import hierarchical_global_local_amd as hg
    L = hg.lib()
    c, cfg = _cfg("c2_decode_heavy", n_kv_heads=kv)
    n = sum(int(np.prod(s)) for _, s, _ in wl.weight_specs(c))
    assert L.bt_weights_bytes(ctypes.byref(cfg)) == n * 2
    assert dict((k, s) for k, s, _ in wl.weight_specs(c))["blk.0.attn.qkv.w"] == (768, 768 + 2 * kv * 64)
    _, mha = _cfg("c2_decode_heavy")
    for which in (0, 1):
        got = []
        for x in (cfg, mha):
            off, nb, cap = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int32()
            assert L.bt_workspace_region(ctypes.byref(x), which, ctypes.byref(off), ctypes.byref(nb),
                                         ctypes.byref(cap)) == 0
            got.append((nb.value, cap.value))
        assert got[0][1] == got[1][1] and got[0][0] * (12 // kv) == got[1][0]


@pytest.mark.parametrize("mode,kw", [("sum", dict()), ("sum", dict(block_len=2)), ("xattn", dict(prefix_len=3)),
                                     ("xattn", dict(n_kv_heads=2))])
def test_context_variant_blob_and_local_cache(mode, kw):
    """Summation projects to L_B vectors and cross-attention adds six tensors per token layer; both
    local caches hold one start slot plus the block's tokens."""
    import hierarchical_global_local_amd as hg
    L = hg.lib()
    c, cfg = _cfg("c2_decode_heavy", context_mode=mode, **kw)
    n = sum(int(np.prod(s)) for _, s, _ in wl.weight_specs(c))
    assert L.bt_weights_bytes(ctypes.byref(cfg)) == n * 2
    assert hg.weight_names(c) == [s[0] for s in wl.weight_specs(c)]
    off, nb, cap = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int32()
    assert L.bt_workspace_region(ctypes.byref(cfg), 1, ctypes.byref(off), ctypes.byref(nb), ctypes.byref(cap)) == 0
    assert cap.value == 1 + c.block_len


def test_paged_pool_sizes_the_block_kv():
    """kv_pages pages of 64 entries (all block layers) replace the per-row caches of full capacity."""
    import hierarchical_global_local_amd as hg
    L = hg.lib()
    c = wl.get_config("c2_decode_heavy")
    flat = hg.BtConfig.make(c, 256, 2180)
    paged = hg.BtConfig.make(c, 256, 2180, kv_pages=1000)
    regions = []
    for cfg in (flat, paged):
        off, nb, cap = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int32()
        assert L.bt_workspace_region(ctypes.byref(cfg), 0, ctypes.byref(off), ctypes.byref(nb), ctypes.byref(cap)) == 0
        regions.append((nb.value, cap.value))
    (flat_b, flat_cap), (paged_b, paged_cap) = regions
    assert flat_cap == 576 and paged_cap == 64
    assert paged_b * 256 * 576 == flat_b * 1000 * 64
    assert L.bt_workspace_bytes(ctypes.byref(paged)) < L.bt_workspace_bytes(ctypes.byref(flat))


def test_context_mode_needs_a_token_decoder():
    import hierarchical_global_local_amd as hg
    _, cfg = _cfg("v2_vanilla_decode_heavy", context_mode="sum")
    assert hg.lib().bt_weights_bytes(ctypes.byref(cfg)) == 0
    assert "token decoder" in hg.lib().bt_last_error().decode()


def test_packed_blob_matches_declared_size():
    import hierarchical_global_local_amd as hg
    c, cfg = _cfg("c0_tiny")
    blob = hg.pack_weights(c, wl.make_weights(c))
    assert blob.nbytes == hg.lib().bt_weights_bytes(ctypes.byref(cfg))


def test_block_kv_footprint_ratio_is_block_len():
    """Block-KV bytes for the 8K-prompt sweep scale as 1/L_B (L_B = 1 is a token-level cache)."""
    import hierarchical_global_local_amd as hg
    sizes = {}
    for name in ("c4_lb1", "c4_lb2", "c4_lb8"):
        c, cfg = _cfg(name)
        off, nb, cap = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int32()
        assert hg.lib().bt_workspace_region(ctypes.byref(cfg), 0, ctypes.byref(off), ctypes.byref(nb),
                                            ctypes.byref(cap)) == 0
        entries = -(-(wl.padded_len(c, c.prompt_len) + c.gen_len) // c.block_len)
        assert cap.value == -(-entries // 64) * 64
        sizes[c.block_len] = entries * nb.value // cap.value
    assert sizes[1] == 2 * sizes[2] == 8 * sizes[8]


@pytest.mark.parametrize("field,value,msg", [("n_heads", 5, "multiple of n_heads"), ("block_len", 0, "block_len"),
                                             ("dtype", 7, "dtype"), ("max_batch", 0, "max_batch"),
                                             ("d_model", 96, "d_head"), ("prefix_len", 40, "prefix_len"),
                                             ("max_prompt_tokens", -4, "max_prompt_tokens"),
                                             ("max_prompt_tokens", 1 << 20, "max_prompt_tokens"),
                                             ("n_kv_heads", 5, "n_kv_heads"), ("n_kv_heads", -1, "n_kv_heads"),
                                             ("n_kv_heads", 24, "n_kv_heads"), ("context_mode", 3, "context_mode"),
                                             ("pad_id", 50304, "pad_id"), ("pad_id", -1, "pad_id"),
                                             ("kv_pages", -1, "kv_pages"), ("kv_pages", 1 << 30, "kv_pages")])
def test_invalid_config_rejected_on_host(field, value, msg):
    import hierarchical_global_local_amd as hg
    _, cfg = _cfg("c1_prefill_heavy")
    setattr(cfg, field, value)
    L = hg.lib()
    assert L.bt_weights_bytes(ctypes.byref(cfg)) == 0
    assert msg in L.bt_last_error().decode()
    assert L.bt_workspace_bytes(ctypes.byref(cfg)) == 0


def test_null_arguments_rejected():
    import hierarchical_global_local_amd as hg
    L = hg.lib()
    assert L.bt_prefill(None, None, 1, 1, None, None) == -1
    assert L.bt_decode_step(None, None, None) == -1
    assert L.bt_destroy(None) == -1


def test_prompt_capacity_sizes_the_activations():
    """max_prompt_tokens bounds the prefill activations (one row per prompt block and batch row);
    the caches still follow max_tokens."""
    import hierarchical_global_local_amd as hg
    c = wl.get_config("c2_decode_heavy")
    Tp = wl.padded_len(c, c.prompt_len)
    full = hg.BtConfig.make(c, 1024, Tp + c.gen_len)
    short = hg.BtConfig.make(c, 1024, Tp + c.gen_len, Tp)
    L = hg.lib()
    nb_full, nb_short = L.bt_workspace_bytes(ctypes.byref(full)), L.bt_workspace_bytes(ctypes.byref(short))
    assert 0 < nb_short < nb_full
    for which in (0, 1):
        got = []
        for cfg in (full, short):
            off, nb, cap = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int32()
            assert L.bt_workspace_region(ctypes.byref(cfg), which, ctypes.byref(off), ctypes.byref(nb),
                                         ctypes.byref(cap)) == 0
            got.append((nb.value, cap.value))
        assert got[0] == got[1]
