"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI binding and compare
with the numpy oracle on the same seeded inputs."""
from __future__ import annotations

import sys
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

import bt_workloads as wl
from oracle import model as om

BF16_TOL = 2e-2   # max-abs logit error, bf16 configs
FP32_TOL = 1e-4   # max-abs logit error, fp32 configs


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device (run them with -m gpu on an MI355X)")
    import hierarchical_global_local_amd as hg
    hg.lib()  # raises if the HIP library is missing: there is no fallback
    return torch


def run_gpu(cfg: wl.Config, W: Dict[str, np.ndarray], prompt: np.ndarray, G: int,
            logits_steps: Iterable[int] = (), max_tokens: Optional[int] = None, max_batch: Optional[int] = None):
    """Greedy generation on the GPU.  Returns (ids [B, G] numpy, {step: logits [B, V] numpy}, model)."""
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    B, T = prompt.shape
    mt = max_tokens or wl.padded_len(cfg, T) + G
    model = hg.BlockTransformer(cfg, W, max_batch=max_batch or B, max_tokens=mt)
    d_prompt = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    ids, logits = model.generate(d_prompt, G, logits_steps)
    torch.cuda.synchronize()
    return ids.cpu().numpy().T.copy(), {g: v.cpu().numpy() for g, v in logits.items()}, model


def check_ids_against(ref_logits: np.ndarray, gpu_ids: np.ndarray, tol: float) -> float:
    """Each GPU id must be an argmax of the oracle's logits up to 2*tol (a wider gap than the
    logit tolerance cannot flip); returns the fraction of exact argmax matches."""
    ref_max = ref_logits.max(axis=-1)
    chosen = np.take_along_axis(ref_logits, gpu_ids[..., None].astype(np.int64), axis=-1)[..., 0]
    bad = chosen < ref_max - 2 * tol
    assert not bad.any(), f"{int(bad.sum())} ids are not within 2*tol of the oracle's maximum"
    return float((om.greedy(ref_logits) == gpu_ids).mean())


def teacher_forced_logits(cfg, W, prompt_row: np.ndarray, gpu_ids_row: np.ndarray, steps: Sequence[int]):
    """Oracle logits of generation steps ``steps`` for one row, on the GPU's id stream."""
    seq = np.concatenate([om.pad_prompt(cfg, prompt_row[None]), gpu_ids_row[None].astype(np.int64)], axis=1)
    Tp = seq.shape[1] - len(gpu_ids_row)
    return om.logits_at(W, cfg, seq, [Tp + g for g in steps])[0]


def sampled_steps(cfg, G: int, every: int = 64) -> list:
    s = set(range(min(G, 2 * cfg.block_len + 1))) | set(range(0, G, every)) | {G - 1}
    return sorted(s)
