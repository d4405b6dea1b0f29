"""Serving-shaped batches on the GPU: a ragged prefill (every row padded only to its own whole
blocks, block-KV lengths of its own) and continuous batching (new sequences take over rows of a
running batch where a block starts).  Rows never interact in the Block Transformer, so each row's
stream must equal the oracle run on that row's prompt alone (fp32: identical ids, 1e-4 logits;
bf16: 2e-2 logits and ids within the tolerance band), and rows that nothing replaced must be bit
for bit what they are without any join."""
import numpy as np
import pytest

import bt_workloads as wl
from oracle import model as om
from tests.gpu_harness import BF16_TOL, FP32_TOL, check_ids_against, log, require_gpu

pytestmark = pytest.mark.gpu

SMALL_BF16 = wl.Config("small_bf16", "bf16", vocab=512, d_model=128, n_heads=2, d_mlp=512, n_block_layers=2,
                       n_token_layers=2, block_len=4, prefix_len=2, batch=5, prompt_len=37, gen_len=20)


def _check_segment(cfg, W64, prompt_row, ids, logits=None):
    """ids [G] generated from prompt_row alone (padded to its own whole blocks) by the GPU."""
    G = len(ids)
    _, ref_lg, st = om.generate(W64, cfg, prompt_row[None], G, keep_logits=True, forced=np.asarray(ids)[None])
    tol = FP32_TOL if cfg.dtype == "fp32" else BF16_TOL
    if cfg.dtype == "fp32":
        np.testing.assert_array_equal(om.greedy(ref_lg[0]), ids)
    else:
        check_ids_against(ref_lg[0], np.asarray(ids), tol)
    if logits is not None:
        err = np.abs(np.stack(logits) - ref_lg[0][: len(logits)]).max()
        assert err <= tol, err
    return st


def _prompts(cfg, B, T, seed):
    rng = np.random.default_rng(seed)
    prompt = rng.integers(0, cfg.vocab, (B, T)).astype(np.int32)   # columns past a row's length are junk
    lengths = rng.integers(1, T + 1, B).astype(np.int32)
    lengths[0] = T
    return prompt, lengths


CASES = {"fp32": lambda: wl.get_config("c0_tiny"), "fp32_lb2": lambda: wl.get_config("c0_tiny", block_len=2),
         "bf16": lambda: SMALL_BF16, "vanilla_fp32": lambda: wl.get_config("c0_tiny", n_token_layers=0, block_len=1)}


@pytest.mark.parametrize("name", list(CASES))
def test_ragged_prefill_matches_each_row_alone(name):
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    cfg = CASES[name]()
    W = wl.make_weights(cfg, seed=31, ln_jitter=True)
    W64 = om.weights_as(W, np.float64)
    B, T, G = 5, 23, 10
    prompt, lengths = _prompts(cfg, B, T, 31)
    log(f"ragged prefill {name}: lengths {lengths.tolist()}")
    model = hg.BlockTransformer(cfg, W, max_batch=B, max_tokens=wl.padded_len(cfg, T) + G)
    ids = torch.empty((G, B), dtype=torch.int32, device="cuda")
    lg = torch.empty((G, B, cfg.vocab), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(model.stream):
        model.prefill(torch.from_numpy(prompt).cuda(), ids[0], lg[0], lengths=torch.from_numpy(lengths).cuda(),
                      ragged=True)
        for g in range(1, G):
            model.decode_step(ids[g], lg[g])
    torch.cuda.synchronize()
    got, glg = ids.cpu().numpy().T, lg.cpu().numpy()
    L = cfg.block_len
    for b in range(B):
        st = _check_segment(cfg, W64, prompt[b, :lengths[b]], got[b], [glg[g, b] for g in range(G)])
        assert st.block_kv_len == -(-int(lengths[b]) // L) + (G - 1) // L
    np.testing.assert_array_equal(model.block_lengths(), [-(-int(n) // L) + (G - 1) // L for n in lengths])


@pytest.mark.parametrize("name", list(CASES))
def test_rows_join_a_running_batch(name):
    """Sequences join at block starts (twice, different rows, different prompt lengths); every row
    segment equals its prompt generated alone; decode steps run from HIP graphs."""
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    cfg = CASES[name]()
    L = cfg.block_len
    W = wl.make_weights(cfg, seed=32, ln_jitter=True)
    W64 = om.weights_as(W, np.float64)
    B, T, steps = 4, 19, 8 * L + 3
    prompt, lengths = _prompts(cfg, B, T, 32)
    joins = {1 + 2 * L: ([1, 3], *_prompts(cfg, 2, 13, 33)), 1 + 5 * L: ([0], *_prompts(cfg, 1, 21, 34))}
    max_tokens = wl.padded_len(cfg, 21) + steps + 1
    log(f"joins {name}: first at {min(joins)}, second at {max(joins)}")

    def run(with_joins):
        model = hg.BlockTransformer(cfg, W, max_batch=B, max_tokens=max(max_tokens, wl.padded_len(cfg, T) + steps))
        segs = [[(prompt[b, :lengths[b]], [])] for b in range(B)]
        with torch.cuda.stream(model.stream):
            out = model.prefill(torch.from_numpy(prompt).cuda(), lengths=torch.from_numpy(lengths).cuda(),
                                ragged=True)
            torch.cuda.synchronize()
            for b, v in enumerate(out.cpu().numpy()):
                segs[b][-1][1].append(int(v))
            for g in range(1, steps):
                if with_joins and g in joins:
                    rows, p, l = joins[g]
                    new = model.join(rows, torch.from_numpy(p).cuda(), torch.from_numpy(l).cuda())
                    torch.cuda.synchronize()
                    for i, r in enumerate(rows):
                        segs[r].append((p[i, :l[i]], [int(new.cpu().numpy()[i])]))
                out = model.decode_step()
                torch.cuda.synchronize()
                for b, v in enumerate(out.cpu().numpy()):
                    segs[b][-1][1].append(int(v))
        return segs, model

    segs, model = run(True)
    for b in range(B):
        for p_row, ids in segs[b]:
            _check_segment(cfg, W64, p_row, ids)
    # rows 2 (never replaced) and the replaced rows before their join: bit-identical to no joins
    base, _ = run(False)
    assert len(segs[2]) == 1 and segs[2][0][1] == base[2][0][1]
    assert segs[1][0][1] == base[1][0][1][: len(segs[1][0][1])]
    # block-KV length of each row: its own prompt blocks plus one per block completed since
    blk = model.block_lengths()
    for b in range(B):
        p_row, ids = segs[b][-1]
        assert blk[b] == -(-len(p_row) // L) + (len(ids) - 1) // L


def test_join_errors_are_reported_on_the_host():
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    cfg = SMALL_BF16
    W = wl.make_weights(cfg, seed=35)
    model = hg.BlockTransformer(cfg, W, max_batch=4, max_tokens=128)
    p = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    l = torch.full((2,), 8, dtype=torch.int32, device="cuda")
    with pytest.raises(hg.BtError, match="before bt_prefill"):
        model.join([0, 1], p, l)
    model.prefill(torch.zeros((4, 9), dtype=torch.int32, device="cuda"))
    with pytest.raises(hg.BtError, match="distinct"):
        model.join([1, 1], p, l)
    with pytest.raises(hg.BtError, match="distinct"):
        model.join([0, 4], p, l)
    model.join([0, 2], p, l)                    # right after the prefill: a block starts
    model.decode_step()
    with pytest.raises(hg.BtError, match="block starts"):
        model.join([0, 1], p, l)
    torch.cuda.synchronize()
    sum_cfg = SMALL_BF16.with_(context_mode="sum")
    m2 = hg.BlockTransformer(sum_cfg, wl.make_weights(sum_cfg, seed=35), max_batch=4, max_tokens=128)
    m2.prefill(torch.zeros((4, 9), dtype=torch.int32, device="cuda"))
    with pytest.raises(hg.BtError, match="BT_CTX_PREFIX"):
        m2.join([0], p[:1], l[:1])
    torch.cuda.synchronize()


def _paged_run(cfg, W, kv_pages, B, T, steps, prompt, lengths, join, with_logits=True):
    """Ragged prefill, decode steps (with logits: launched eagerly; without: replayed from graphs),
    one join at `join[0]`; returns ids, logits, model."""
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    model = hg.BlockTransformer(cfg, W, max_batch=B, max_tokens=wl.padded_len(cfg, T) + steps + 1,
                                kv_pages=kv_pages)
    ids, lgs = [], []
    with torch.cuda.stream(model.stream):
        lg = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
        ids.append(model.prefill(torch.from_numpy(prompt).cuda(), logits=lg,
                                 lengths=torch.from_numpy(lengths).cuda(), ragged=True).clone())
        lgs.append(lg.clone())
        for g in range(1, steps):
            if g == join[0]:
                rows, p, l = join[1:]
                ids.append(model.join(rows, torch.from_numpy(p).cuda(), torch.from_numpy(l).cuda()).clone())
            lg = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda") if with_logits else None
            ids.append(model.decode_step(logits=lg).clone())
            if with_logits:
                lgs.append(lg.clone())
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ids], [t.cpu().numpy() for t in lgs], model


@pytest.mark.parametrize("name", ["fp32", "bf16"])
def test_paged_block_kv_is_bit_identical_to_flat(name):
    """Pages of 64 entries from a shared pool instead of one cache per row: rows spanning several
    pages, decode steps that open new pages, and a join that hands pages back and takes new
    ones give exactly the flat cache's ids and logits."""
    cfg = (wl.get_config("c0_tiny") if name == "fp32" else SMALL_BF16).with_(block_len=1, prefix_len=2)
    W = wl.make_weights(cfg, seed=36, ln_jitter=True)
    B, T, steps = 4, 150, 90
    prompt, lengths = _prompts(cfg, B, T, 36)
    lengths[1], lengths[2] = 64, 63                       # a row ending exactly at a page boundary
    join = (40, [2], *_prompts(cfg, 1, 100, 37))
    flat = _paged_run(cfg, W, 0, B, T, steps, prompt, lengths, join)
    paged = _paged_run(cfg, W, 14, B, T, steps, prompt, lengths, join)   # flat: 4 rows x 4 pages
    for a, b in zip(flat[0], paged[0]):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(flat[1], paged[1]):
        np.testing.assert_array_equal(a, b)
    replayed = _paged_run(cfg, W, 14, B, T, steps, prompt, lengths, join, with_logits=False)
    for a, b in zip(flat[0], replayed[0]):
        np.testing.assert_array_equal(a, b)
    n = paged[2].block_lengths()
    np.testing.assert_array_equal(n, flat[2].block_lengths())
    tab = paged[2].page_table()
    held = [tab[b, : -(-int(n[b]) // 64)].tolist() for b in range(B)]
    allp = sum(held, [])
    assert len(allp) == len(set(allp)), "a page is held by two rows"
    log(f"paged {name}: block lengths {n.tolist()}, pages {held}")


def test_paged_block_kv_one_wave_per_unit_is_bit_identical_to_flat():
    """1024 ragged rows x 2 heads (2048 units): the block attention's one-wave-per-unit mode reads and
    appends through the page table and gives exactly the flat cache's ids and logits."""
    cfg = SMALL_BF16.with_(block_len=1, prefix_len=2)
    W = wl.make_weights(cfg, seed=38, ln_jitter=True)
    B, T, steps = 1024, 70, 60
    prompt, lengths = _prompts(cfg, B, T, 38)
    flat = _paged_run(cfg, W, 0, B, T, steps, prompt, lengths, (-1,))
    paged = _paged_run(cfg, W, 3 * B, B, T, steps, prompt, lengths, (-1,))   # capacity: 3 pages a row
    for a, b in zip(flat[0], paged[0]):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(flat[1], paged[1]):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(paged[2].block_lengths(), flat[2].block_lengths())
    log(f"paged one-wave mode: block lengths {int(paged[2].block_lengths().min())}.."
        f"{int(paged[2].block_lengths().max())}")


def test_paged_pool_exhaustion_is_a_host_error():
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    cfg = SMALL_BF16.with_(block_len=1, prefix_len=2)
    W = wl.make_weights(cfg, seed=38)
    model = hg.BlockTransformer(cfg, W, max_batch=2, max_tokens=400, kv_pages=4)
    p = torch.zeros((2, 130), dtype=torch.int32, device="cuda")
    l = torch.tensor([130, 60], dtype=torch.int32, device="cuda")
    model.prefill(p, lengths=l, ragged=True)            # 3 + 1 pages: the pool is full
    with pytest.raises(hg.BtError, match="kv_pages exhausted"):
        for _ in range(10):                             # row 1 needs a new page at 64 entries
            model.decode_step()
    torch.cuda.synchronize()
    with pytest.raises(hg.BtError, match="kv_pages exhausted"):
        model.prefill(torch.zeros((2, 300), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
