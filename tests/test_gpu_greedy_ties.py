"""Greedy ids on exact ties.  The classifier's rows repeat with period 64 (row j is row j mod 64), so
every logit value is attained by several ids that fall in different column slabs and workgroups, and
the greedy rule (the lowest id among equal maxima, the oracle's argmax) must always pick an id below
64.  The three classifier kernels each meet it: the skinny kernel (up to 64 rows), the 128 x 128
LDS-tiled kernel (65-128 rows) and the 256 x 128 kernel (above 128 rows), each followed by the
two-stage reduction of the per-workgroup maxima.  fp32 compares every id with the oracle's."""
import numpy as np
import pytest

import bt_workloads as wl
from oracle import model as om
from tests.gpu_harness import BF16_TOL, FP32_TOL, check_ids_against, log, run_gpu
from tests.test_gpu_parity import SMALL_BF16

pytestmark = pytest.mark.gpu

PERIOD = 64


def _tied_weights(cfg, seed):
    W = wl.make_weights(cfg, seed=seed, ln_jitter=True)
    head = W["head.w"]
    W["head.w"] = np.ascontiguousarray(head[np.arange(head.shape[0]) % PERIOD])
    return W


def test_ties_fp32_every_step():
    cfg = wl.get_config("c0_tiny")
    B, T, G = 3, 13, 12
    W = _tied_weights(cfg, seed=21)
    prompt = wl.make_prompt(cfg, batch=B, T=T, seed=21)
    ids, lg, _ = run_gpu(cfg, W, prompt, G, logits_steps=range(G))
    ref_ids, ref_lg, _ = om.generate(om.weights_as(W, np.float64), cfg, prompt, G, keep_logits=True)
    gl = np.stack([lg[g] for g in range(G)], axis=1)
    err = float(np.abs(gl - ref_lg).max())
    log(f"fp32 ties: max-abs logit error {err:.2e}, ids {np.unique(ids)[:8]}...")
    assert err <= FP32_TOL
    assert (ids < PERIOD).all()
    np.testing.assert_array_equal(ids, ref_ids)


@pytest.mark.parametrize("B", [5, 100, 200])
def test_ties_bf16_each_classifier_kernel(B):
    cfg = SMALL_BF16.with_(batch=B, prompt_len=9, gen_len=9)
    G = cfg.gen_len
    W = _tied_weights(cfg, seed=22)
    prompt = wl.make_prompt(cfg, seed=22)
    ids, lg, _ = run_gpu(cfg, W, prompt, G, logits_steps=range(G))
    gl = np.stack([lg[g] for g in range(G)], axis=1)
    # the GPU's logits repeat exactly with the rows: the ties the rule decides are real on the GPU
    np.testing.assert_array_equal(gl[..., PERIOD:2 * PERIOD], gl[..., :PERIOD])
    _, ref_lg, _ = om.generate(om.weights_as(W, np.float64), cfg, prompt, G, keep_logits=True, forced=ids)
    err = float(np.abs(gl - ref_lg).max())
    exact = check_ids_against(ref_lg, ids, BF16_TOL)
    log(f"bf16 ties B={B}: max-abs logit error {err:.2e}, exact argmax {exact:.3f}")
    assert err <= BF16_TOL
    assert (ids < PERIOD).all()
