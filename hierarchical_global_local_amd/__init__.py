"""Block Transformer batched inference on one MI355X (gfx950).

A thin ctypes binding over libbt.so (include/bt.h): it marshals arguments and
owns device memory through PyTorch tensors; every step of the inference path
runs in the library's HIP kernels.  Importing this package does not load the
library; the first use does, and fails loudly if it has not been built
(``python -m hierarchical_global_local_amd.build`` or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, List, Mapping, Optional, Sequence

import numpy as np

__all__ = ["BtConfig", "BlockTransformer", "lib", "pack_weights", "weight_names", "BtError",
           "BT_FP32", "BT_BF16", "PROFILE_KINDS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
# BT_LIBRARY names another build of the same library (for instance one with host sanitizers)
_LIB_PATH = os.environ.get("BT_LIBRARY") or os.path.join(_PKG, "libbt.so")

BT_FP32, BT_BF16 = 0, 1
# bt_context_mode values of the workload names
CONTEXT_MODES = {"prefix": 0, "sum": 1, "xattn": 2}

PROFILE_KINDS = ["embed", "layernorm", "gemm_qkv_up", "gemm_out_down", "gemm_prefix", "gemm_head",
                 "attn_prefill", "rope_scatter", "attn_block_decode", "attn_local", "finalize", "attn_cross",
                 "local_attn_out"]


class BtError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libbt error {code}: {msg}")
        self.code = code


class BtConfig(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_mlp", ctypes.c_int32), ("n_block_layers", ctypes.c_int32), ("n_token_layers", ctypes.c_int32),
                ("block_len", ctypes.c_int32), ("prefix_len", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32), ("pad_id", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("rope_base", ctypes.c_float), ("max_prompt_tokens", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("context_mode", ctypes.c_int32), ("kv_pages", ctypes.c_int32)]

    @classmethod
    def make(cls, model, max_batch: int, max_tokens: int, max_prompt_tokens: int = 0,
             kv_pages: int = 0) -> "BtConfig":
        """From any object with the model fields (vocab, d_model, ..., dtype "fp32"/"bf16")."""
        return cls(model.vocab, model.d_model, model.n_heads, model.d_mlp, model.n_block_layers,
                   model.n_token_layers, model.block_len, model.prefix_len, max_batch, max_tokens,
                   BT_FP32 if model.dtype == "fp32" else BT_BF16, model.pad_id, model.ln_eps, model.rope_base,
                   max_prompt_tokens, getattr(model, "n_kv_heads", 0),
                   CONTEXT_MODES[getattr(model, "context_mode", "prefix")], kv_pages)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libbt.so; raises if it was not built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build the HIP library first "
                          "(python -m hierarchical_global_local_amd.build)")
    L = ctypes.CDLL(_LIB_PATH)
    c_p, c_i32, c_sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(BtConfig)
    L.bt_weights_bytes.argtypes, L.bt_weights_bytes.restype = [cfgp], c_sz
    L.bt_workspace_bytes.argtypes, L.bt_workspace_bytes.restype = [cfgp], c_sz
    L.bt_init.argtypes = [cfgp, c_p, c_p, c_sz, c_p, ctypes.POINTER(c_p)]
    L.bt_prefill.argtypes = [c_p, c_p, c_i32, c_i32, c_p, c_p]
    L.bt_prefill_lengths.argtypes = [c_p, c_p, c_p, c_i32, c_i32, c_p, c_p]
    L.bt_prefill_ragged.argtypes = [c_p, c_p, c_p, c_i32, c_i32, c_p, c_p]
    L.bt_prefill_rows.argtypes = [c_p, ctypes.POINTER(c_i32), c_i32, c_p, c_p, c_i32, c_p, c_p]
    L.bt_block_lengths.argtypes = [c_p, ctypes.POINTER(c_i32)]
    L.bt_page_table.argtypes = [c_p, ctypes.POINTER(c_i32)]
    L.bt_decode_step.argtypes = [c_p, c_p, c_p]
    L.bt_decode_step_static.argtypes = [c_p, c_p, c_p]
    L.bt_cache_lengths.argtypes = [c_p, ctypes.POINTER(c_i32), ctypes.POINTER(c_i32)]
    L.bt_workspace_region.argtypes = [cfgp, c_i32, ctypes.POINTER(c_sz), ctypes.POINTER(c_sz), ctypes.POINTER(c_i32)]
    L.bt_destroy.argtypes = [c_p]
    L.bt_last_error.argtypes, L.bt_last_error.restype = [], ctypes.c_char_p
    L.bt_profile_enable.argtypes = [c_p, c_i32]
    dp = ctypes.POINTER(ctypes.c_double)
    L.bt_profile_read.argtypes = [c_p, c_i32, dp, ctypes.POINTER(ctypes.c_int64), dp, dp]
    L.bt_test_gemm.argtypes = [c_i32, c_p, c_p, c_p, c_i32, c_i32, c_i32, ctypes.c_float, c_p]
    L.bt_set_graphs.argtypes = [c_p, c_i32]
    L.bt_test_replay.argtypes = [c_p, c_i32, c_i32]
    L.bt_test_fuse_local.argtypes = [c_p, c_i32]
    L.bt_numerics_status.argtypes = [c_p, c_i32, ctypes.POINTER(ctypes.c_int64)]
    for f in ("bt_init", "bt_prefill", "bt_prefill_lengths", "bt_prefill_ragged", "bt_prefill_rows",
              "bt_block_lengths", "bt_page_table", "bt_decode_step", "bt_decode_step_static", "bt_cache_lengths", "bt_workspace_region", "bt_destroy",
              "bt_profile_enable", "bt_profile_read", "bt_test_gemm", "bt_set_graphs", "bt_test_replay",
              "bt_test_fuse_local", "bt_numerics_status"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def check(code: int) -> None:
    if code != 0:
        raise BtError(code, lib().bt_last_error().decode())


def weight_names(model) -> List[str]:
    """Canonical tensor names in weights-blob order (include/bt.h)."""
    layer = ["ln1.g", "ln1.b", "attn.qkv.w", "attn.qkv.b", "attn.out.w", "attn.out.b", "ln2.g", "ln2.b",
             "mlp.up.w", "mlp.up.b", "mlp.down.w", "mlp.down.b"]
    names = ["emb_block"]
    names += [f"blk.{l}.{n}" for l in range(model.n_block_layers) for n in layer]
    names += ["blk.lnf.g", "blk.lnf.b"]
    if model.n_token_layers == 0:  # token-level transformer
        return names + ["head.w"]
    names += ["prefix.w", "prefix.b", "emb_token"]
    xattn = ["xattn.q.w", "xattn.q.b", "xattn.kv.w", "xattn.kv.b", "xattn.out.w", "xattn.out.b"]
    tok_layer = layer + (xattn if getattr(model, "context_mode", "prefix") == "xattn" else [])
    names += [f"tok.{l}.{n}" for l in range(model.n_token_layers) for n in tok_layer]
    names += ["tok.lnf.g", "tok.lnf.b", "head.w"]
    return names


def pack_weights(model, weights: Mapping[str, np.ndarray]) -> np.ndarray:
    """Concatenate the parameters into the canonical blob (uint8), fp32 or bf16 (round to nearest even)."""
    import torch
    parts = []
    for name in weight_names(model):
        a = torch.from_numpy(np.ascontiguousarray(weights[name], dtype=np.float32)).reshape(-1)
        if model.dtype == "bf16":
            a = a.to(torch.bfloat16)
        parts.append(a.view(torch.uint8))
    return torch.cat(parts).numpy()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class BlockTransformer:
    """One model instance bound to a CUDA/HIP stream.  Device memory is owned by torch tensors."""

    def __init__(self, model, weights: Mapping[str, np.ndarray], max_batch: int, max_tokens: int,
                 device: str = "cuda:0", stream=None, graphs: bool = True, max_prompt_tokens: int = 0,
                 kv_pages: int = 0):
        import torch
        self.torch = torch
        L = lib()
        self.model = model
        self.cfg = BtConfig.make(model, max_batch, max_tokens, max_prompt_tokens, kv_pages)
        self.device = torch.device(device)
        # a stream of its own: decode steps are captured into HIP graphs, which the NULL stream forbids
        self.stream = stream if stream is not None else torch.cuda.Stream(self.device)
        wbytes = L.bt_weights_bytes(ctypes.byref(self.cfg))
        if wbytes == 0:
            raise BtError(-1, L.bt_last_error().decode())
        blob = pack_weights(model, weights)
        if blob.nbytes != wbytes:
            raise BtError(-1, f"packed weights are {blob.nbytes} bytes, the library expects {wbytes}")
        ws_bytes = L.bt_workspace_bytes(ctypes.byref(self.cfg))
        with torch.cuda.stream(self.stream):
            d_blob = torch.from_numpy(blob).to(self.device)
            self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        check(L.bt_init(ctypes.byref(self.cfg), d_blob.data_ptr(), self.workspace.data_ptr(), ws_bytes,
                        self.stream.cuda_stream, ctypes.byref(h)))
        self.stream.synchronize()
        del d_blob
        self.h = h
        self.batch = 0
        check(L.bt_set_graphs(self.h, 1 if graphs else 0))

    def close(self) -> None:
        if getattr(self, "h", None):
            lib().bt_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ inference
    def _order(self, *tensors) -> None:
        """Make the library's stream wait for work already queued on the caller's current stream,
        and tell torch's allocator that the tensors are used on the library's stream."""
        cur = self.torch.cuda.current_stream(self.device)
        if cur != self.stream:
            self.stream.wait_stream(cur)
            for t in tensors:
                if t is not None:
                    t.record_stream(self.stream)

    def prefill(self, prompt, out=None, logits=None, lengths=None, ragged=False):
        """prompt: int32 device tensor [B, T]; writes the first generated ids into ``out`` [B].
        lengths: optional int32 device tensor [B]: row b's prompt is prompt[b, :lengths[b]], left
        padded to the common length (bt_prefill_lengths) or, with ragged=True, only to its own
        whole blocks (bt_prefill_ragged)."""
        torch = self.torch
        assert prompt.dtype == torch.int32 and prompt.is_contiguous() and prompt.dim() == 2
        B, T = prompt.shape
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=self.device)
        if lengths is None:
            self._order(prompt, out, logits)
            check(lib().bt_prefill(self.h, prompt.data_ptr(), B, T, out.data_ptr(), _ptr(logits)))
        else:
            assert lengths.dtype == torch.int32 and lengths.is_contiguous() and lengths.shape == (B,)
            self._order(prompt, lengths, out, logits)
            fn = lib().bt_prefill_ragged if ragged else lib().bt_prefill_lengths
            check(fn(self.h, prompt.data_ptr(), lengths.data_ptr(), B, T, out.data_ptr(), _ptr(logits)))
        self.batch = B
        return out

    def join(self, rows, prompt, lengths, out=None, logits=None):
        """Continuous batching (bt_prefill_rows): the prompts of ``prompt`` [B_new, T] / ``lengths``
        [B_new] (int32 device tensors) take over rows ``rows`` (host ints) of the running batch.
        Returns their first generated ids [B_new]."""
        torch = self.torch
        assert prompt.dtype == torch.int32 and prompt.is_contiguous() and prompt.dim() == 2
        Bn, T = prompt.shape
        assert lengths.dtype == torch.int32 and lengths.is_contiguous() and lengths.shape == (Bn,)
        if out is None:
            out = torch.empty(Bn, dtype=torch.int32, device=self.device)
        self._order(prompt, lengths, out, logits)
        r = (ctypes.c_int32 * Bn)(*[int(x) for x in rows])
        check(lib().bt_prefill_rows(self.h, r, Bn, prompt.data_ptr(), lengths.data_ptr(), T, out.data_ptr(),
                                    _ptr(logits)))
        return out

    def page_table(self):
        """Paged block KV: the page table [max_batch][cap / 64] (synchronises)."""
        blocks = -(-self.cfg.max_tokens // self.model.block_len)
        a = (ctypes.c_int32 * (self.cfg.max_batch * -(-blocks // 64)))()
        check(lib().bt_page_table(self.h, a))
        return np.array(a, dtype=np.int64).reshape(self.cfg.max_batch, -1)

    def block_lengths(self):
        """Block-KV entries of every row of the running batch (synchronises)."""
        a = (ctypes.c_int32 * self.batch)()
        check(lib().bt_block_lengths(self.h, a))
        return np.array(a, dtype=np.int64)

    def decode_step(self, out=None, logits=None):
        torch = self.torch
        if out is None:
            out = torch.empty(self.batch, dtype=torch.int32, device=self.device)
        self._order(out, logits)
        check(lib().bt_decode_step(self.h, out.data_ptr(), _ptr(logits)))
        return out

    def decode_step_static(self, out=None, logits=None):
        """One decode step through bt_decode_step_static: no allocation, no graph of its own, the
        step's partial results in the library's static scratch (see include/bt.h)."""
        torch = self.torch
        if out is None:
            out = torch.empty(self.batch, dtype=torch.int32, device=self.device)
        self._order(out, logits)
        check(lib().bt_decode_step_static(self.h, out.data_ptr(), _ptr(logits)))
        return out

    def set_graphs(self, enable: bool) -> None:
        check(lib().bt_set_graphs(self.h, 1 if enable else 0))

    def set_fuse_local(self, enable: bool) -> None:
        """Decode steps with the token decoder's local attention inside its [out|down] GEMM (default)
        or as a launch of its own (see bt_test_fuse_local in include/bt_test.h)."""
        check(lib().bt_test_fuse_local(self.h, 1 if enable else 0))

    def generate(self, prompt, G: int, logits_steps: Iterable[int] = ()):
        """Greedy generation of G tokens: ids [G, B] (device int32) and {step: logits [B, V] fp32}."""
        torch = self.torch
        B = prompt.shape[0]
        steps = set(int(s) for s in logits_steps)
        ids = torch.empty((G, B), dtype=torch.int32, device=self.device)
        logits: Dict[int, "torch.Tensor"] = {}
        with torch.cuda.stream(self.stream):
            for g in range(G):
                lg = None
                if g in steps:
                    lg = torch.empty((B, self.model.vocab), dtype=torch.float32, device=self.device)
                    logits[g] = lg
                if g == 0:
                    self.prefill(prompt, ids[0], lg)
                else:
                    self.decode_step(ids[g], lg)
        return ids, logits

    # ------------------------------------------------------------------ introspection
    def cache_lengths(self):
        a, b = ctypes.c_int32(), ctypes.c_int32()
        check(lib().bt_cache_lengths(self.h, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def cache_view(self, which: int):
        """Block-KV (which=0) or local-KV (1) region as a typed tensor view, plus its per-head capacity."""
        torch = self.torch
        off, nb, cap = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int32()
        check(lib().bt_workspace_region(ctypes.byref(self.cfg), which, ctypes.byref(off), ctypes.byref(nb),
                                        ctypes.byref(cap)))
        dt = torch.float32 if self.model.dtype == "fp32" else torch.float16
        raw = self.workspace[off.value: off.value + nb.value]
        return raw.view(dt), cap.value

    def numerics_status(self, reset: bool = False) -> dict:
        """bt_numerics_status: weight elements rounded at init, and whether an activation or cache
        value was clamped to fp16's range since the flag was last cleared (synchronises)."""
        a = (ctypes.c_int64 * 2)()
        check(lib().bt_numerics_status(self.h, 1 if reset else 0, a))
        return {"weights_rounded": int(a[0]), "values_clamped": bool(a[1])}

    def profile(self, on: bool) -> None:
        check(lib().bt_profile_enable(self.h, 1 if on else 0))

    def replay(self, kind: str, reps: int) -> None:
        """Launch the decode kernel of class `kind` ("gemm_qkv_up", "attn_block_decode",
        "local_attn_out", or "empty" for a kernel that does nothing) `reps` times back to back on the
        model's stream (see bt_test_replay in include/bt_test.h)."""
        check(lib().bt_test_replay(self.h, -1 if kind == "empty" else PROFILE_KINDS.index(kind), reps))

    def profile_read(self) -> Dict[str, dict]:
        """{phase/kind: {"ms", "launches", "bytes", "flops"}} since profile(True); phase is prefill or decode."""
        n = 2 * len(PROFILE_KINDS)
        ms, by, fl = (ctypes.c_double * n)(), (ctypes.c_double * n)(), (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        check(lib().bt_profile_read(self.h, n, ms, cnt, by, fl))
        out = {}
        for i in range(n):
            phase = "prefill" if i < len(PROFILE_KINDS) else "decode"
            name = f"{phase}/{PROFILE_KINDS[i % len(PROFILE_KINDS)]}"
            out[name] = {"ms": ms[i], "launches": cnt[i], "bytes": by[i], "flops": fl[i]}
        return out


def gemm(a, w, M: int, N: int, K: int, scale: float = 1.0, stream=None):
    """C [M, N] = scale * A @ W.T in fp32 through the library's GEMM kernels.  a, w: fp32 row-major
    [M, K] / [N, K] device tensors, or fp16 device tensors already in the library's operand order
    (see bt_test_gemm in include/bt_test.h)."""
    import torch
    assert a.dtype == w.dtype and a.dtype in (torch.float32, torch.float16)
    assert a.is_contiguous() and w.is_contiguous()
    rows_a = M if a.dtype == torch.float32 else (M + 15) // 16 * 16
    assert a.numel() == rows_a * K and w.numel() == N * K
    c = torch.empty((M, N), dtype=torch.float32, device=a.device)
    st = stream if stream is not None else torch.cuda.current_stream(a.device)
    check(lib().bt_test_gemm(BT_FP32 if a.dtype == torch.float32 else BT_BF16, a.data_ptr(), w.data_ptr(),
                             c.data_ptr(), M, N, K, scale, st.cuda_stream))
    return c
