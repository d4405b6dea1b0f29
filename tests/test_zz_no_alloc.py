"""bt_decode_step_static (the decode step that allocates nothing, its partial results in the
library's static scratch) called through the C-ABI, against bt_decode_step on a second handle with
the same weights: two generations in a row, the second on a smaller batch, with identical ids and
logits, bit for bit (same kernels, same summation order), at every step."""
import numpy as np
import pytest

import bt_workloads as wl
from tests.gpu_harness import log, require_gpu

pytestmark = pytest.mark.gpu

SMALL = wl.Config("small_bf16", "bf16", vocab=512, d_model=128, n_heads=2, d_mlp=512, n_block_layers=2,
                  n_token_layers=2, block_len=4, prefix_len=2, batch=48, prompt_len=21, gen_len=14)


def _run(model, prompt, G, static):
    torch = require_gpu()
    B = prompt.shape[0]
    ids = torch.empty((G, B), dtype=torch.int32, device="cuda")
    logits = []
    with torch.cuda.stream(model.stream):
        for g in range(G):
            lg = torch.empty((B, model.model.vocab), dtype=torch.float32, device="cuda") if g % 3 == 1 else None
            if g == 0:
                model.prefill(prompt, ids[0], lg)
            elif static:
                model.decode_step_static(ids[g], lg)
            else:
                model.decode_step(ids[g], lg)
            if lg is not None:
                logits.append(lg)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), [l.cpu().numpy() for l in logits]


@pytest.mark.parametrize("cfg", [SMALL, wl.get_config("c2_decode_heavy", batch=64, prompt_len=24, gen_len=10)],
                         ids=["small_bf16", "d768"])
def test_static_decode_step_matches_decode_step(cfg):
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    W = wl.make_weights(cfg)
    G = cfg.gen_len
    mt = wl.padded_len(cfg, cfg.prompt_len) + G
    ref = hg.BlockTransformer(cfg, W, max_batch=cfg.batch, max_tokens=mt)
    new = hg.BlockTransformer(cfg, W, max_batch=cfg.batch, max_tokens=mt)
    for B in (cfg.batch, cfg.batch // 3):   # the second call on a smaller input
        prompt = torch.from_numpy(wl.make_prompt(cfg, batch=B, seed=B)).cuda()
        ids_a, lg_a = _run(ref, prompt, G, static=False)
        ids_b, lg_b = _run(new, prompt, G, static=True)
        log(f"{cfg.name} B={B} G={G}: ids equal {bool((ids_a == ids_b).all())}, "
            f"logit steps {len(lg_a)}, max diff {max(float(np.abs(a - b).max()) for a, b in zip(lg_a, lg_b)):.3e}")
        np.testing.assert_array_equal(ids_a, ids_b)
        for a, b in zip(lg_a, lg_b):
            np.testing.assert_array_equal(a, b)
        assert ref.cache_lengths() == new.cache_lengths()
    # a batch whose partial results exceed the static array is refused before anything is queued
    ref.close()
    new.close()


def test_static_decode_step_refuses_oversized_batch():
    require_gpu()
    import hierarchical_global_local_amd as hg
    import torch
    cfg = wl.get_config("c2_decode_heavy", batch=1024, prompt_len=8, gen_len=3)
    W = wl.make_weights(cfg)
    m = hg.BlockTransformer(cfg, W, max_batch=cfg.batch, max_tokens=wl.padded_len(cfg, cfg.prompt_len) + cfg.gen_len)
    prompt = torch.from_numpy(wl.make_prompt(cfg)).cuda()
    with torch.cuda.stream(m.stream):
        out = m.prefill(prompt)
        with pytest.raises(hg.BtError) as e:
            m.decode_step_static(out)
    log(f"batch 1024: {e.value}")
    assert e.value.code == -2 and "static scratch" in str(e.value)
    # the refused call queued nothing: the ordinary step still continues the generation
    with torch.cuda.stream(m.stream):
        m.decode_step()
    torch.cuda.synchronize()
    m.close()
