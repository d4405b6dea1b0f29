"""Range of the fp16 values of the BT_BF16 path: weight matrices are held as fp16 scaled by 2^8, so
bt_init must refuse a weight fp16 cannot hold (magnitude >= 256, or not finite), count the weights
it rounds (magnitudes below 2^-25 that are not multiples of 2^-32), and activations or cache values beyond fp16's range
must be flagged when they are clamped (bt_numerics_status)."""
import numpy as np
import pytest

import bt_workloads as wl
from tests.gpu_harness import log, require_gpu

pytestmark = pytest.mark.gpu

SMALL = wl.Config("small_bf16", "bf16", vocab=512, d_model=128, n_heads=2, d_mlp=512, n_block_layers=2,
                  n_token_layers=2, block_len=4, prefix_len=2, batch=3, prompt_len=13, gen_len=9)


def _model(cfg, W):
    import hierarchical_global_local_amd as hg
    return hg.BlockTransformer(cfg, W, max_batch=cfg.batch, max_tokens=wl.padded_len(cfg, cfg.prompt_len) + cfg.gen_len)


def _generate(model, cfg):
    torch = require_gpu()
    prompt = torch.from_numpy(wl.make_prompt(cfg)).cuda()
    ids, _ = model.generate(prompt, cfg.gen_len)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


@pytest.mark.parametrize("name,value", [("blk.1.mlp.down.w", 300.0), ("head.w", -256.0), ("prefix.w", np.inf),
                                        ("tok.0.attn.qkv.w", np.nan)])
def test_weight_beyond_fp16_is_rejected(name, value):
    """A single weight of magnitude >= 256 (or inf / NaN) makes bt_init fail with
    BT_ERR_UNSUPPORTED and name the tensor; no handle is created."""
    require_gpu()
    import hierarchical_global_local_amd as hg
    W = wl.make_weights(SMALL)
    W[name] = W[name].copy()
    W[name][3, 5] = value
    with pytest.raises(hg.BtError) as e:
        _model(SMALL, W)
    log(f"{name} = {value}: {e.value}")
    assert e.value.code == -5 and name in str(e.value)


def test_largest_and_smallest_exact_weights_accepted():
    """255 (the largest bf16 below 256), 2^-25 with a full mantissa (1.9921875 * 2^-25) and 2^-30
    (a multiple of 2^-32) convert exactly: accepted, nothing rounded.  (1 + 2^-7) * 2^-30 and
    1.5 * 2^-33 are not multiples of 2^-32 (fp16's spacing below 2^-14 is 2^-24, 2^-32 before the
    2^8 pre-scale): accepted and counted as rounded, once per planted element."""
    require_gpu()
    W = wl.make_weights(SMALL)
    W["blk.0.attn.out.w"] = W["blk.0.attn.out.w"].copy()
    W["blk.0.attn.out.w"][0, 0] = 255.0
    W["blk.0.attn.out.w"][1, 1] = -1.9921875 * 2.0 ** -25
    W["blk.0.attn.out.w"][2, 2] = 2.0 ** -30
    m = _model(SMALL, W)
    st = m.numerics_status(reset=True)
    log(f"exact extremes: {st}")
    assert st["weights_rounded"] == 0
    m.close()
    W["tok.1.mlp.up.w"] = W["tok.1.mlp.up.w"].copy()
    W["tok.1.mlp.up.w"][2, 7] = (1.0 + 2.0 ** -7) * 2.0 ** -30
    W["tok.1.mlp.up.w"][4, 9] = -1.5 * 2.0 ** -33
    m = _model(SMALL, W)
    st = m.numerics_status(reset=True)
    log(f"two tiny weights: {st}")
    assert st["weights_rounded"] == 2
    m.close()


def test_activation_clamp_flag():
    """A random-init model never leaves fp16's range (flag clear after a generation); LayerNorm
    gains of 1e5 push the normalised operands past 65504, and the flag reports the clamp until it
    is cleared."""
    require_gpu()
    W = wl.make_weights(SMALL)
    m = _model(SMALL, W)
    m.numerics_status(reset=True)
    _generate(m, SMALL)
    st = m.numerics_status(reset=True)
    log(f"random init: {st}")
    assert st == {"weights_rounded": 0, "values_clamped": False}
    m.close()
    for k in [k for k in W if k.endswith("ln1.g")]:
        W[k] = np.full_like(W[k], 1e5)
    m = _model(SMALL, W)
    m.numerics_status(reset=True)
    ids = _generate(m, SMALL)
    st = m.numerics_status(reset=False)
    log(f"LayerNorm gains 1e5: {st}")
    assert st["values_clamped"] and ((ids >= 0) & (ids < SMALL.vocab)).all()
    assert m.numerics_status(reset=True)["values_clamped"]
    assert not m.numerics_status(reset=False)["values_clamped"]
    m.close()
