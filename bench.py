"""Throughput benchmark of Block Transformer batched inference on one MI355X.

One step = one greedy generation over the batch: bt_prefill of the whole prompt, then G-1
bt_decode_step calls (the whole hot path: embedder, block decoder, prefix, token decoder,
classifier).  Inputs are resident in HBM before the timed region starts.  Prints one JSON line.

Workloads (synthetic random-init weights N(0, 0.02^2), uniform random prompt ids):
  c1_prefill_heavy  d=768, 6+6 layers, L_B=4, P=1, V=50304, batch 64, 2048-token prompt, 128 generated
  c2_decode_heavy   same model, batch 256, 128-token prompt, 2048 generated (reported alongside)
The default line also carries the roofline of the dominant kernel class, the token-level
transformers of the same shapes on the same kernels, a batch sweep of the decode-heavy shape, and
the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "generated tokens/sec @1 MI355X (prefill- & decode-heavy); decode HBM GB/s"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 / bf16 MFMA, TFLOP/s


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic cost model
# The minimal traffic and arithmetic of the method itself (summary page "Block Transformer:
# Global-to-Local Language Modeling for Fast Inference", §3.4 "The Inference Cost Model": decode is
# bound by reading parameters and KV caches, prefill by compute): every weight read once per decode
# step for the whole batch, every cached KV entry read once per use, activations passed between
# kernels not counted; prefill FLOPs of the linear maps, the causal block attention, the prefix pass
# and the classifier of the first token.

def _layer_params(cfg, token_layer=False):
    """Weights and biases of one layer (q|k|v, out, up, down, two LayerNorms; the cross-attention
    branch of a token layer)."""
    D, F = cfg.d_model, cfg.d_mlp
    kvw = cfg.kv_heads * cfg.d_head
    qw = D + 2 * kvw
    n = D * qw + qw + D * D + D + 2 * D * F + F + D + 4 * D
    if token_layer and cfg.context_mode == "xattn":
        n += D * D + D + D * 2 * kvw + 2 * kvw + D * D + D
    return n


def _layer_matmul_params(cfg):
    """Weights of the matrices one row of a block layer multiplies (flops = 2 x this per row)."""
    D, F = cfg.d_model, cfg.d_mlp
    return D * (D + 2 * cfg.kv_heads * cfg.d_head) + D * D + 2 * D * F


def decode_bytes_parts(cfg, G=None):
    """Algorithmic bytes of the G - 1 decode steps of a generation of G tokens, by kind: a step at
    in-block offset j reads the token decoder's weights, the final LayerNorm and the classifier once
    ("weights"), each row's token embedding ("embeddings") and its P + j local entries per token
    layer ("local_kv"); a block step (j = 0) also reads the block decoder's weights, the context
    projection, each row's block embedding, the n + 1 block-KV entries per block layer ("block_kv",
    n cached before the step) and the P new prefix entries per token layer."""
    G = cfg.gen_len if G is None else G
    w = 2 if cfg.dtype == "bf16" else 4
    D, V, B, L = cfg.d_model, cfg.vocab, cfg.batch, cfg.block_len
    kv = 2 * cfg.kv_heads * cfg.d_head                     # K and V elements of one entry
    Nb, Nt, lead, NC = cfg.n_block_layers, cfg.n_token_layers, cfg.lead, cfg.n_ctx
    n0 = -(-max(cfg.prompt_len, L) // L)                   # prompt blocks after left padding
    head = 2 * D + V * D
    parts = {"weights": 0, "embeddings": 0, "local_kv": 0, "block_kv": 0}
    for g in range(1, G):
        j = g % L
        if Nt:
            parts["weights"] += w * (Nt * _layer_params(cfg, True) + head)
            parts["embeddings"] += B * w * D
            parts["local_kv"] += B * w * Nt * kv * (lead + j)
        if j == 0:
            n = n0 + g // L - 1
            parts["weights"] += w * (Nb * _layer_params(cfg) + (0 if Nt else head) +
                                     (2 * D + D * NC * D + NC * D if Nt else 0))
            parts["embeddings"] += B * w * D
            parts["block_kv"] += B * w * Nb * kv * (n + 1)
            parts["local_kv"] += B * w * Nt * kv * lead
    return parts


def decode_bytes(cfg, G=None):
    """Algorithmic bytes of the G - 1 decode steps of a generation of G tokens (decode_bytes_parts)."""
    return sum(decode_bytes_parts(cfg, G).values())


def prefill_flops(cfg):
    """Algorithmic FLOPs of a prefill: the block decoder's linear maps over every prompt block and
    its causal attention, the token decoder over the prefix slots, the classifier of one token."""
    D, V, B, L = cfg.d_model, cfg.vocab, cfg.batch, cfg.block_len
    n = -(-max(cfg.prompt_len, L) // L)
    Nb, Nt = cfg.n_block_layers, cfg.n_token_layers
    f = 2 * B * n * Nb * _layer_matmul_params(cfg) + Nb * B * 4 * D * (n * (n + 1) // 2)
    if Nt:
        f += 2 * B * cfg.lead * Nt * _layer_matmul_params(cfg) + 2 * B * D * cfg.n_ctx * D
    return f + 2 * B * V * D


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def describe(cfg):
    return (f"{cfg.name}: Block Transformer d={cfg.d_model} {cfg.n_block_layers}+{cfg.n_token_layers} layers "
            f"H={cfg.n_heads}{'' if cfg.kv_heads == cfg.n_heads else f' H_kv={cfg.kv_heads}'} MLP={cfg.d_mlp} "
            f"L_B={cfg.block_len} P={cfg.prefix_len} V={cfg.vocab}"
            f"{'' if cfg.context_mode == 'prefix' else f' context={cfg.context_mode}'}, "
            f"batch {cfg.batch}, {cfg.prompt_len}-token prompt, {cfg.gen_len} generated")


class Runner:
    def __init__(self, cfg, prompt_sized=False, W=None):
        """prompt_sized: size the prefill activations for this prompt only (max_prompt_tokens), as a
        server that knows its longest prompt would; the caches are sized for prompt + generation.
        W: the model's weights if already drawn (wl.make_weights(cfg))."""
        import torch

        import bt_workloads as wl
        import hierarchical_global_local_amd as hg
        self.torch, self.cfg = torch, cfg
        self.G = cfg.gen_len
        if W is None:
            W = wl.make_weights(cfg)
        prompt = wl.make_prompt(cfg)
        Tp = wl.padded_len(cfg, cfg.prompt_len)
        self.model = hg.BlockTransformer(cfg, W, max_batch=cfg.batch, max_tokens=Tp + self.G,
                                         max_prompt_tokens=Tp if prompt_sized else 0)
        del W
        self.stream = self.model.stream
        self.prompt = torch.from_numpy(prompt).cuda()
        self.ids = torch.empty((self.G, cfg.batch), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

    def step(self, ev=None):
        """One generation; optional events mark (start, after prefill, end) on the model's stream."""
        if ev:
            ev[0].record(self.stream)
        self.model.prefill(self.prompt, self.ids[0])
        if ev:
            ev[1].record(self.stream)
        for g in range(1, self.G):
            self.model.decode_step(self.ids[g])
        if ev:
            ev[2].record(self.stream)

    def timed(self, steps, warmup):
        torch = self.torch
        with torch.cuda.stream(self.stream):
            for _ in range(warmup):
                self.step()
            torch.cuda.synchronize()
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
            t0 = time.perf_counter()
            for e in evs:
                self.step(e)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        pre = [e[0].elapsed_time(e[1]) for e in evs]
        dec = [e[1].elapsed_time(e[2]) for e in evs]
        tot = [e[0].elapsed_time(e[2]) for e in evs]
        return dict(wall_s=wall, ms_per_step=sum(tot) / steps, prefill_ms=sum(pre) / steps,
                    decode_ms=sum(dec) / steps)

    def replay_us(self, kind, reps):
        """Average duration of one launch of a decode kernel class, launched `reps` times back to back
        (bt_test_replay) between HIP events on the model's stream."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        self.model.replay(kind, 10)
        e0.record(self.stream)
        self.model.replay(kind, reps)
        e1.record(self.stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def profiled(self, steps):
        """Repeat the timed steps with HIP events around every launch: per-class time, bytes, flops."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            self.model.profile(True)
            t0 = time.perf_counter()
            for _ in range(steps):
                self.step()
            prof = self.model.profile_read()
            wall = time.perf_counter() - t0
            self.model.profile(False)
        for v in prof.values():
            for k in ("ms", "launches", "bytes", "flops"):
                v[k] /= steps
        return prof, wall / steps * 1e3


def classify(name):
    """Roofline of a kernel class: prefill GEMMs and prefill attention are MFMA contractions, the rest
    (all decode kernels, gathers, norms, scatters) move bytes."""
    phase, kind = name.split("/")
    if phase == "prefill" and (kind.startswith("gemm") or kind == "attn_prefill"):
        return "mfma"
    return "hbm"


REPLAYABLE = {"decode/gemm_qkv_up": "gemm_qkv_up", "decode/local_attn_out": "local_attn_out",
              "decode/attn_block_decode": "attn_block_decode"}


def attn_replay_roofline(runner, cfg):
    """Block-attention decode at the block-KV length reached at the end of the generation: K and V of
    n entries read once per (row, KV head), q|k|v read, the new entry and the output written (fp16)."""
    n, _ = runner.model.cache_lengths()
    reps = 20 * cfg.n_block_layers
    us = runner.replay_us("attn_block_decode", reps)
    D, B, kvw = cfg.d_model, cfg.batch, cfg.kv_heads * cfg.d_head
    per_launch = B * n * kvw * 2 * 2 + B * (2 * D + 4 * kvw) * 2
    achieved = per_launch / (us * 1e-6) / 1e9
    tr = stored_traffic("decode/attn_block_decode")
    return {"kernel_class": "decode/attn_block_decode", "bound": "hbm", "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": round(tr["traffic_bytes_per_launch"], 1) if tr and tr.get("workload") == cfg.name else None,
            "block_kv_entries": n, "avg_launch_us": round(us, 3), "algorithmic_per_launch": per_launch,
            "measured": f"HIP events around {reps} back-to-back launches (bt_test_replay) at n = {n}"}


def roofline_of(name, rec):
    bound = classify(name)
    if bound == "mfma":
        achieved = rec["flops"] / (rec["ms"] * 1e-3) / 1e12
        peak, unit = MFMA_F16_PEAK_TFLOPS, "TFLOP/s"
        per_launch = rec["flops"] / max(rec["launches"], 1)
    else:
        achieved = rec["bytes"] / (rec["ms"] * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
        per_launch = rec["bytes"] / max(rec["launches"], 1)
    return {"kernel_class": name, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None, "launches_per_step": rec["launches"],
            "avg_launch_us": round(rec["ms"] * 1e3 / max(rec["launches"], 1), 3),
            "algorithmic_per_launch": per_launch}


COPY_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
def traffic_json(kernel_class):
    """Counter-measured traffic of a decode kernel class, e.g. profiles/traffic_decode_gemm_qkv_up.json."""
    return os.path.join(PROFILES, "traffic_" + kernel_class.replace("/", "_") + ".json")


def _rocprof_db(d):
    import glob
    found = glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True)
    if not found:
        raise FileNotFoundError(f"no rocprofv3 results database under {d}")
    return found[0]


def summarize_rocprof(d, top=25, run=32):
    """Per-kernel totals of a rocprofv3 --kernel-trace run (the same figures --stats reports), then,
    for the kernels with the most time, the launches made back to back (runs of at least `run`
    consecutive dispatches of the same kernel: bt_test_replay) separated from those inside the
    generation steps."""
    import sqlite3
    cur = sqlite3.connect(_rocprof_db(d)).cursor()
    rows = list(cur.execute("select name, count(*), sum(end-start), avg(end-start), min(end-start), max(end-start) "
                            "from kernels group by name order by sum(end-start) desc"))
    total = sum(r[2] for r in rows)
    out = [f"{'total_ms':>10} {'pct':>6} {'calls':>7} {'avg_us':>9} {'min_us':>9} {'max_us':>9}  kernel"]
    for name, n, tot, avg, mn, mx in rows[:top]:
        out.append(f"{tot / 1e6:10.3f} {100 * tot / total:6.2f} {n:7d} {avg / 1e3:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f}  {name[:140]}")
    seq = list(cur.execute("select name, end - start from kernels order by start"))
    groups, i = {}, 0
    while i < len(seq):
        j = i
        while j < len(seq) and seq[j][0] == seq[i][0]:
            j += 1
        key = "back_to_back" if j - i >= run else "in_step"
        g = groups.setdefault(seq[i][0], {"in_step": [], "back_to_back": []})
        g[key] += [t for _, t in seq[i:j]]
        i = j
    out.append(f"# launches in runs of >= {run} consecutive dispatches of one kernel (back to back) vs the rest:")
    out.append(f"{'in_step_calls':>13} {'in_step_avg_us':>14} {'b2b_calls':>9} {'b2b_avg_us':>10}  kernel")
    for name, *_ in rows[:8]:
        g = groups[name]
        a, bb = g["in_step"], g["back_to_back"]
        out.append(f"{len(a):13d} {sum(a) / max(len(a), 1) / 1e3:14.2f} {len(bb):9d} "
                   f"{(sum(bb) / len(bb) / 1e3 if bb else 0.0):10.2f}  {name[:140]}")
    return "\n".join(out)


def mfma_from_counters(d, n_xcc=8, n_simd=1024):
    """Per-kernel MFMA work and busy fraction from a rocprofv3 --pmc run with SQ_INSTS_VALU_MFMA_MOPS_F16,
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (one aggregated value per dispatch and counter):
    flops = MOPS x 512 (the counter counts multiply-add operations / 512); GRBM_GUI_ACTIVE is summed
    over the 8 XCDs, so the dispatch's clock cycles are GUI_ACTIVE / 8 (and / duration, the clock);
    the busy cycles are summed over the 1024 SIMDs, so busy fraction = BUSY / (cycles x 1024)."""
    import sqlite3
    cur = sqlite3.connect(_rocprof_db(d)).cursor()
    per = {}
    for kname, disp, cname, value, dur in cur.execute(
            "select kernel_name, dispatch_id, counter_name, sum(value), max(duration) from counters_collection "
            "group by dispatch_id, counter_name"):
        e = per.setdefault(kname, {}).setdefault(disp, {"duration_ns": float(dur)})
        e[cname] = float(value)
    res = []
    for kname, disps in per.items():
        v = list(disps.values())
        mops = sum(x.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) for x in v)
        if not mops:
            continue
        busy = sum(x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for x in v)
        cyc = sum(x.get("GRBM_GUI_ACTIVE", 0.0) for x in v) / n_xcc
        dur = sum(x["duration_ns"] for x in v)
        n = len(v)
        res.append({"kernel": kname, "dispatches": n, "mfma_flops_per_dispatch": 512.0 * mops / n,
                    "avg_duration_us": dur / n / 1e3, "tflops": 512.0 * mops / (dur * 1e-9) / 1e12,
                    "clock_ghz": cyc / dur, "mfma_busy": busy / max(cyc * n_simd, 1.0)})
    res.sort(key=lambda r: -r["mfma_flops_per_dispatch"] * r["dispatches"])
    return res


def _counter_per_dispatch(d, counter):
    import sqlite3
    cur = sqlite3.connect(_rocprof_db(d)).cursor()
    rows = cur.execute("select kernel_name, counter_name, value from counters_collection")
    per = {}
    for kname, cname, value in rows:
        if cname.startswith(counter):
            per.setdefault(kname, []).append(float(value))
    return per


# the source file holding each replayable kernel class and its launch configuration
CLASS_SOURCE = {"decode/gemm_qkv_up": "gemm_decode.hip", "decode/local_attn_out": "gemm_decode.hip",
                "decode/attn_block_decode": "attention.hip"}


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_text(path):
    """A source file's code without its comments, trailing blanks and empty lines (string and
    character literals kept whole): what decides the compiled kernels, so that a stored counter
    result outlives an edit of the comments but not one of the code."""
    with open(path) as f:
        src = f.read()
    src = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", src)
    return "\n".join(l.rstrip() for l in src.splitlines() if l.strip()).encode()


def source_hash(kernel_class):
    """Hash of the kernel's source code and of the build flags: stored counter results are used only
    while both are unchanged."""
    import hashlib
    h = hashlib.sha256()
    h.update(code_text(os.path.join(ROOT, "hierarchical_global_local_amd", "csrc", CLASS_SOURCE[kernel_class])))
    from hierarchical_global_local_amd import build as _b
    # the code-generation flags only: include paths name this checkout's location
    h.update(" ".join(f for f in _b.FLAGS if not f.startswith("-I")).encode())
    return h.hexdigest()[:16]


def traffic_from_counters(fetch_dir, write_dir, kernel_pattern, kernel_class, workload, command):
    """Average HBM bytes per dispatch of the kernel matching kernel_pattern (of class kernel_class),
    from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for the 1 GiB reference copy (--copy-calibration).  Written to profiles/ with the hash of the
    kernel's source and the build flags."""
    fetch, write = _counter_per_dispatch(fetch_dir, "FETCH_SIZE"), _counter_per_dispatch(write_dir, "WRITE_SIZE")
    copy_f = next(v for k, v in fetch.items() if "copy" in k.lower() or "elementwise" in k.lower())
    copy_w = next(v for k, v in write.items() if "copy" in k.lower() or "elementwise" in k.lower())
    f_scale = COPY_BYTES / (max(copy_f) * 1024.0)
    w_scale = COPY_BYTES / (max(copy_w) * 1024.0)
    names = [k for k in fetch if kernel_pattern in k]
    if not names:
        raise KeyError(f"no kernel matches {kernel_pattern}")
    name = names[0]
    fb = sum(fetch[name]) / len(fetch[name]) * 1024.0 * f_scale
    wb = sum(write[name]) / len(write[name]) * 1024.0 * w_scale
    res = {"kernel": name, "dispatches": len(fetch[name]), "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
           "traffic_bytes_per_launch": fb + wb, "fetch_scale": f_scale, "write_scale": w_scale,
           "kernel_class": kernel_class, "workload": workload, "source_sha256_16": source_hash(kernel_class)}
    os.makedirs(PROFILES, exist_ok=True)
    out_json = traffic_json(kernel_class)
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    # readable summary of the two counter runs next to it
    lines = [f"# HBM traffic of the {kernel_class} kernel ({name[:60]}...) in {workload}",
             "# commands (two passes, one counter each; the 1 GiB reference copy precedes the workload):",
             "#   cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT"]
    for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        lines.append(f"#   rocprofv3 --pmc {c} -d {d} -o run -- {command}")
    lines.append(f"#   python bench.py --traffic {fetch_dir} {write_dir} --kernel {kernel_pattern} --kernel-class {kernel_class} "
                 f"--workload {workload} --command '{command}'")
    lines.append(f"# scaling: FETCH_SIZE of the 1 GiB copy reads {max(copy_f):.0f} KiB (x{f_scale:.3f}), "
                 f"WRITE_SIZE {max(copy_w):.0f} KiB (x{w_scale:.3f})")
    lines.append("# per-kernel averages (KiB per dispatch, unscaled), the 10 most frequent kernels:")
    for cname, d in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        for k, vs in sorted(d.items(), key=lambda kv: -len(kv[1]))[:10]:
            lines.append(f"{cname}  {len(vs):6d}  {sum(vs) / len(vs):10.1f}  {k[:110]}")
    lines.append(f"# result ({os.path.relpath(out_json, ROOT)}): fetch {fb / 1e6:.2f} MB + write {wb / 1e6:.2f} MB "
                 f"per launch = {(fb + wb) / 1e6:.2f} MB")
    # every decode kernel of the generation, for the decode phase's counter-measured rate
    import bt_workloads as wl
    cfg = wl.get_config(workload)
    ds = decode_step_traffic(fetch_dir, write_dir, workload, f_scale, w_scale, cfg.gen_len - 1)
    lines.append(f"# all {ds['dispatches']} decode dispatches of the generation ({ds['decode_steps']} steps, every kernel): "
                 f"fetch {ds['fetch_bytes'] / 1e9:.2f} GB + write {ds['write_bytes'] / 1e9:.2f} GB = "
                 f"{ds['traffic_bytes'] / 1e9:.2f} GB (profiles/traffic_decode_steps.json)")
    with open(os.path.join(PROFILES, "counters_" + kernel_class.replace("/", "_") + "_" + workload + ".txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return res


def _decode_phase_kib(d, counter):
    """Sum of a counter (KiB) over the dispatches of the decode steps of one generation: those
    after the prefill's greedy-id finalisation (the first k_finalize dispatch), and their count."""
    import sqlite3
    cur = sqlite3.connect(_rocprof_db(d)).cursor()
    rows = list(cur.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection "
                            "order by dispatch_id"))
    first = min(r[0] for r in rows if "k_finalize" in r[1])
    sel = [r for r in rows if r[0] > first and r[2].startswith(counter)]
    return sum(float(r[3]) for r in sel), len({r[0] for r in sel})


def all_sources_hash():
    """Hash of the code of every library source and header and of the code-generation flags."""
    import hashlib
    from hierarchical_global_local_amd import build as _b
    h = hashlib.sha256()
    for fn in sorted(os.listdir(os.path.join(ROOT, "hierarchical_global_local_amd", "csrc"))):
        h.update(code_text(os.path.join(ROOT, "hierarchical_global_local_amd", "csrc", fn)))
    h.update(" ".join(f for f in _b.FLAGS if not f.startswith("-I")).encode())
    return h.hexdigest()[:16]


def decode_step_traffic(fetch_dir, write_dir, workload, f_scale, w_scale, steps):
    """HBM bytes of all decode steps of one generation (every kernel, counter-measured), stored for
    the benchmark line's decode_counter_gbps."""
    fk, nf = _decode_phase_kib(fetch_dir, "FETCH_SIZE")
    wk, nw = _decode_phase_kib(write_dir, "WRITE_SIZE")
    res = {"workload": workload, "decode_steps": steps, "dispatches": nf, "fetch_bytes": fk * 1024.0 * f_scale,
           "write_bytes": wk * 1024.0 * w_scale, "traffic_bytes": fk * 1024.0 * f_scale + wk * 1024.0 * w_scale,
           "fetch_scale": f_scale, "write_scale": w_scale, "source_sha256_16": all_sources_hash()}
    with open(os.path.join(PROFILES, "traffic_decode_steps.json"), "w") as f:
        json.dump(res, f, indent=1)
    return res


def stored_decode_step_traffic(workload):
    """The counter-measured bytes of all decode steps of one generation of `workload`, or None if
    absent, taken on another workload, or taken before any library source or flag changed."""
    try:
        with open(os.path.join(PROFILES, "traffic_decode_steps.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ok = t.get("workload") == workload and t.get("source_sha256_16") == all_sources_hash()
    return t if ok else None


def trace_in_step_us(workload, kernel_name):
    """Average in-step duration (us) of a kernel in the committed trace summary of the workload's
    bench command (profiles/kernels_<workload>.txt: launches outside back-to-back replays), or None."""
    try:
        with open(os.path.join(PROFILES, f"kernels_{workload}.txt")) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    try:
        start = next(i for i, l in enumerate(lines) if l.lstrip().startswith("in_step_calls"))
    except StopIteration:
        return None
    for l in lines[start + 1:]:
        parts = l.split()
        if len(parts) == 5 and kernel_name.startswith(parts[4]) and int(parts[0]) > 0:
            return float(parts[1])
    return None


def stored_traffic(kernel_class):
    """Counter-measured bytes per launch of a decode kernel class, or None if absent or if the
    kernel's source or the build flags changed since the counters were taken."""
    if kernel_class not in CLASS_SOURCE:
        return None
    try:
        with open(traffic_json(kernel_class)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("source_sha256_16") == source_hash(kernel_class) else None


def cpu_baseline(cfg, rows, tokens):
    """The oracle (numpy fp32, incremental prefill + decode) on a bounded sample of the workload."""
    import numpy as np

    import bt_workloads as wl
    from oracle import model as om
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=1)
    except Exception:
        threads = os.cpu_count() or 1
    W = om.weights_as(wl.make_weights(cfg), np.float32)
    prompt = wl.make_prompt(cfg)[:rows]
    t0 = time.perf_counter()
    om.generate(W, cfg, prompt, tokens)
    dt = time.perf_counter() - t0
    return {"value": round(rows * tokens / dt, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{cfg.name}: rows 0..{rows - 1} of the batch, full {cfg.prompt_len}-token prompt, "
                      f"{tokens} generated tokens (numpy fp32 incremental path), {dt:.1f} s wall",
            "host": cpu_model(), "host_cpus": os.cpu_count(), "blas_threads": int(threads)}


def sweep_points(base, batches, van=None, van_batches=(), cache=None):
    """Generated tokens/s against batch size at one prompt / generation shape (the pages measure
    both models at their largest batch and report batch sensitivity).  Workspaces are sized for the
    prompt (max_prompt_tokens) so that the batch is bounded by the caches; one untimed and one
    timed generation per point.  cache: {(model name, batch): tokens/s} measured elsewhere in this
    run, reused instead of measured again."""
    import torch

    import bt_workloads as wl
    rows = []
    for cfg0, bs in ((base, batches), (van, van_batches)):
        if cfg0 is None or not bs:
            continue
        W = wl.make_weights(cfg0)
        for B in bs:
            cfg = cfg0.with_(batch=int(B))
            rec = {"model": cfg0.name, "batch": int(B)}
            if cache and (cfg0.name, int(B)) in cache:
                rec.update(cache[(cfg0.name, int(B))])
                rec["note"] = "measured above in this run"
            else:
                try:
                    r = Runner(cfg, prompt_sized=True, W=W)
                    t = r.timed(1, 1)
                    rec.update(tokens_per_s=round(cfg.batch * cfg.gen_len / (t["ms_per_step"] * 1e-3), 1),
                               ms_per_step=round(t["ms_per_step"], 2), prefill_ms=round(t["prefill_ms"], 2),
                               decode_ms=round(t["decode_ms"], 2),
                               workspace_gib=round(r.model.workspace.numel() / 2 ** 30, 2))
                    del r
                except torch.cuda.OutOfMemoryError:
                    rec["result"] = "does not fit in HBM"
                torch.cuda.empty_cache()
            log(f"[sweep] {rec}")
            rows.append(rec)
        del W
    return rows


def batch_sweep(args):
    import bt_workloads as wl
    base = wl.get_config(args.sweep_config)
    van = None
    if args.sweep_vanilla:
        van = wl.get_config({"c2_decode_heavy": "v2_vanilla_decode_heavy",
                             "c1_prefill_heavy": "v1_vanilla_prefill_heavy"}[args.sweep_config])
    rows = sweep_points(base, [int(b) for b in args.batch_sweep.split(",")], van,
                        [int(b) for b in args.sweep_vanilla.split(",")] if args.sweep_vanilla else ())
    line = json.dumps({"batch_sweep": describe(base), "gen_len": base.gen_len, "prompt_len": base.prompt_len,
                       "points": rows})
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


# The pages' headline claim, restated (context only: other hardware, trained models, batch sizes not given).
PAGES_CLAIM = {
    "claim": "Block Transformer inference throughput 10 to 20 times that of vanilla (token-level) transformers "
             "of equal perplexity, at the largest batch that fits in memory, prefill-heavy and decode-heavy",
    "hardware": "NVIDIA H100 (throughput comparison), a single H100 for the wall-time breakdown; precision not stated",
    "source": "summary page 'Block Transformer: Global-to-Local Language Modeling for Fast Inference', "
              "abstract and §5 Main Quantitative Results (throughput comparison)",
}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c1_prefill_heavy")
    ap.add_argument("--decode-config", default="c2_decode_heavy", help="second workload reported alongside, or 'none'")
    ap.add_argument("--cpu-rows", type=int, default=16)
    ap.add_argument("--cpu-tokens", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device-to-device twice (reference kernel for HBM counter scaling)")
    ap.add_argument("--summarize", metavar="ROCPROF_DIR", help="print a kernel summary of a rocprofv3 run and exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="HBM traffic of the dominant kernel from two rocprofv3 --pmc runs; writes profiles/")
    ap.add_argument("--mfma", metavar="ROCPROF_DIR",
                    help="per-kernel MFMA flops and busy fraction of a rocprofv3 --pmc run and exit")
    ap.add_argument("--kernel", default=None, help="kernel-name pattern for --traffic")
    ap.add_argument("--kernel-class", default="decode/gemm_qkv_up", help="kernel class of --kernel")
    ap.add_argument("--workload", default="c1_prefill_heavy", help="workload of the --traffic counter runs")
    ap.add_argument("--command", default="", help="the bench command the --traffic counter runs profiled")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the token-level (vanilla) comparison and the batch sweep of the default line")
    ap.add_argument("--compare-batches", default="1,64,1024,4096",
                    help="batch sizes of the Block Transformer in the default line's sweep (decode-heavy shape)")
    ap.add_argument("--compare-vanilla-batches", default="1,64,256,1024",
                    help="batch sizes of the token-level model in the default line's sweep")
    ap.add_argument("--batch-sweep", default=None, metavar="B1,B2,...",
                    help="only sweep the batch size of --sweep-config (one untimed + one timed generation each) "
                         "and print one JSON line; with --sweep-vanilla also the token-level model")
    ap.add_argument("--sweep-config", default="c2_decode_heavy")
    ap.add_argument("--sweep-vanilla", default=None, metavar="B1,B2,...",
                    help="batch sizes of the token-level model of the same shape for --batch-sweep")
    ap.add_argument("--no-profile", action="store_true",
                    help="skip the event-profiled repeat (roofline null); for hardware-counter runs")
    args = ap.parse_args()
    if args.summarize:
        print(summarize_rocprof(args.summarize))
        return
    if args.mfma:
        print(f"{'calls':>7} {'GFLOP/call':>11} {'avg_us':>9} {'TFLOP/s':>8} {'GHz':>5} {'busy':>6}  kernel")
        for r in mfma_from_counters(args.mfma):
            print(f"{r['dispatches']:7d} {r['mfma_flops_per_dispatch'] / 1e9:11.3f} {r['avg_duration_us']:9.2f} "
                  f"{r['tflops']:8.1f} {r['clock_ghz']:5.2f} {r['mfma_busy']:6.3f}  {r['kernel'][:110]}")
        return
    if args.traffic:
        print(json.dumps(traffic_from_counters(args.traffic[0], args.traffic[1], args.kernel, args.kernel_class,
                                               args.workload, args.command), indent=1))
        return
    if args.batch_sweep:
        batch_sweep(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the Block Transformer path shards by batch rows with no "
              "exchange (each GPU would run this same step on its own rows); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import bt_workloads as wl
    if args.copy_calibration:
        a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(2):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    cfg = wl.get_config(args.config)
    log(f"[bench] {describe(cfg)}")
    r = Runner(cfg)
    t = r.timed(args.steps, args.warmup)
    log(f"[bench] timed {args.steps} steps: {t['ms_per_step']:.2f} ms/step "
        f"(prefill {t['prefill_ms']:.2f} ms, decode {t['decode_ms']:.2f} ms)")
    B, G = cfg.batch, cfg.gen_len
    value = B * G / (t["ms_per_step"] * 1e-3)
    dec_gbps = decode_bytes(cfg) / (t["decode_ms"] * 1e-3) / 1e9
    pre_tf = prefill_flops(cfg) / (t["prefill_ms"] * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t["ms_per_step"], 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 weights, fp16 MFMA operands",
        "compute": "bf16 weights held as fp16 after a 2^8 pre-scale (exact for magnitudes in [2^-25, 256)); matrix "
                   "operands and KV caches fp16; fp32 accumulation, softmax, LayerNorm and residual stream",
        "data": "synthetic (random-init N(0,0.02^2) weights, uniform random prompt ids)",
        "config": {"workload": describe(cfg), "global_batch": B, "seq_len": cfg.prompt_len, "gen_len": G},
        "prefill_ms": round(t["prefill_ms"], 3), "decode_ms": round(t["decode_ms"], 3),
        "prefill_tflops": round(pre_tf, 2), "prefill_mfma_frac": round(pre_tf / MFMA_F16_PEAK_TFLOPS, 4),
        "decode_hbm_gbps": round(dec_gbps, 1), "decode_hbm_frac": round(dec_gbps / HBM_PEAK_GBS, 4),
        "rates_from": "algorithmic prefill FLOPs and decode bytes (weights once per step, KV once per use, no "
                      "inter-kernel activations) over the timed phase durations",
        "roofline": None,
    }
    ds = stored_decode_step_traffic(cfg.name)
    if ds is not None:
        # every decode kernel's counter-measured HBM bytes (FETCH_SIZE + WRITE_SIZE of one generation,
        # stored by --traffic) over the decode phase timed here
        cg = ds["traffic_bytes"] / (t["decode_ms"] * 1e-3) / 1e9
        result["decode_counter_gbps"] = round(cg, 1)
        result["decode_counter_frac"] = round(cg / HBM_PEAK_GBS, 4)
        result["decode_counter_source"] = ("profiles/traffic_decode_steps.json: FETCH_SIZE + WRITE_SIZE over the "
                                           f"{ds['dispatches']} decode dispatches of one generation "
                                           f"({ds['traffic_bytes'] / 1e9:.2f} GB)")
    if not args.no_profile:
        prof, prof_ms = r.profiled(args.steps)
        active = {k: v for k, v in prof.items() if v["launches"]}
        dominant = max(active, key=lambda k: active[k]["ms"])
        classes = {k: {"ms_per_step": round(v["ms"], 3), "launches": v["launches"],
                       "rate": roofline_of(k, v)["achieved"], "unit": roofline_of(k, v)["unit"]}
                   for k, v in sorted(active.items(), key=lambda kv: -kv[1]["ms"])}
        for k, v in classes.items():
            log(f"[bench]   {k:28s} {v['ms_per_step']:9.3f} ms/step  {v['launches']:8.1f} launches  {v['rate']:9.1f} {v['unit']}")
        result["roofline"] = roofline_of(dominant, prof[dominant])
        result["roofline"]["measured"] = ("HIP events on the library's stream around every launch of the class, "
                                          f"over a profiled repeat of the {args.steps} timed steps")
        if dominant in REPLAYABLE:
            # per-launch events add their own dispatch latency to short kernels: time the same kernel
            # launched back to back instead, its operands cycled so that none is cache-resident from
            # the previous launch (as inside a step)
            reps = 30 * (cfg.n_token_layers + cfg.n_block_layers)
            us = r.replay_us(REPLAYABLE[dominant], reps)
            roof = result["roofline"]
            roof["event_avg_launch_us_in_steps"] = roof["avg_launch_us"]
            roof["avg_launch_us"] = round(us, 3)
            rate = roof["algorithmic_per_launch"] / (us * 1e-6)
            roof["achieved"] = round(rate / 1e9 if roof["unit"] == "GB/s" else rate / 1e12, 2)
            roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
            # the fixed cost of one dependent launch on the same stream (an empty kernel launched back to
            # back): even a kernel that moved its bytes at peak bandwidth would last this long plus
            # bytes / peak, which bounds the fraction one launch of this size can reach
            floor = r.replay_us("empty", reps)
            roof["launch_floor_us"] = round(floor, 3)
            per = roof["algorithmic_per_launch"]
            peak_rate = roof["peak"] * (1e9 if roof["unit"] == "GB/s" else 1e12)
            roof["frac_ceiling_at_floor"] = round(per / (floor * 1e-6 + per / peak_rate) / peak_rate, 4)
            roof["measured"] = (f"HIP events on the library's stream around {reps} back-to-back launches of the "
                                f"class's kernel at the decode shape (bt_test_replay: weights cycled over all layers "
                                f"of both decoders, activation operand cycled over distinct rows), after the timed "
                                f"steps; algorithmic bytes per launch from the profiled repeat of the timed steps")
        tr = stored_traffic(dominant)
        if tr is not None:
            # the same kernel's in-step average from the committed trace of this command (taken with
            # the counters, on the same kernel source): the duration inside the generation steps
            tus = trace_in_step_us(cfg.name, tr["kernel"])
            if tus is not None:
                roof = result["roofline"]
                peak_rate = roof["peak"] * (1e9 if roof["unit"] == "GB/s" else 1e12)
                roof["in_step_trace_avg_launch_us"] = tus
                roof["in_step_trace_frac"] = round(roof["algorithmic_per_launch"] / (tus * 1e-6) / peak_rate, 4)
                roof["in_step_trace_source"] = f"profiles/kernels_{cfg.name}.txt"
            result["roofline"]["traffic"] = round(tr["traffic_bytes_per_launch"], 1)
            result["roofline"]["traffic_source"] = (os.path.relpath(traffic_json(dominant), ROOT) +
                                                    " (FETCH_SIZE + WRITE_SIZE)")
        result["profiled_ms_per_step"] = round(prof_ms, 3)
        result["kernel_classes"] = classes
    del r
    torch.cuda.empty_cache()
    measured = {(cfg.name, cfg.batch): {"tokens_per_s": round(value, 1)}}
    if args.decode_config != "none":
        c2 = wl.get_config(args.decode_config)
        log(f"[bench] {describe(c2)}")
        r2 = Runner(c2)
        t2 = r2.timed(1, 1)
        prof2, _ = r2.profiled(1)
        dom2 = max((k for k in prof2 if prof2[k]["launches"]), key=lambda k: prof2[k]["ms"])
        d2_gbps = decode_bytes(c2) / (t2["decode_ms"] * 1e-3) / 1e9
        v2 = c2.batch * c2.gen_len / (t2["ms_per_step"] * 1e-3)
        result["decode_heavy"] = {
            "workload": describe(c2), "value": round(v2, 1),
            "unit": "tokens/s", "ms_per_step": round(t2["ms_per_step"], 3),
            "prefill_ms": round(t2["prefill_ms"], 3), "decode_ms": round(t2["decode_ms"], 3),
            "decode_tokens_per_s": round(c2.batch * (c2.gen_len - 1) / (t2["decode_ms"] * 1e-3), 1),
            "decode_hbm_gbps": round(d2_gbps, 1), "decode_hbm_frac": round(d2_gbps / HBM_PEAK_GBS, 4),
            "block_attn_decode": attn_replay_roofline(r2, c2),
            "dominant": roofline_of(dom2, prof2[dom2]),
        }
        measured[(c2.name, c2.batch)] = {"tokens_per_s": round(v2, 1)}
        log(f"[bench] decode-heavy: {v2:.0f} tokens/s, decode {d2_gbps:.1f} GB/s")
        del r2
        torch.cuda.empty_cache()
    if not args.no_compare:
        # the pages' headline comparison: token-level transformers of the same width and total depth
        # on the same kernels, at the prefill-heavy shape and over the decode-heavy batch sweep
        van1 = wl.get_config("v1_vanilla_prefill_heavy")
        rr = Runner(van1)
        tt = rr.timed(1, 1)
        v1 = van1.batch * van1.gen_len / (tt["ms_per_step"] * 1e-3)
        del rr
        torch.cuda.empty_cache()
        log(f"[bench] {van1.name}: {v1:.0f} tokens/s")
        base, van = wl.get_config("c2_decode_heavy"), wl.get_config("v2_vanilla_decode_heavy")
        pts = sweep_points(base, [int(b) for b in args.compare_batches.split(",")] + [base.batch], van,
                           [int(b) for b in args.compare_vanilla_batches.split(",")], cache=measured)
        blk = {p["batch"]: p["tokens_per_s"] for p in pts if p["model"] == base.name and "tokens_per_s" in p}
        vtk = {p["batch"]: p["tokens_per_s"] for p in pts if p["model"] == van.name and "tokens_per_s" in p}
        cmp = {"prefill_heavy": {"block": round(value, 1), "vanilla": round(v1, 1),
                                 "block_over_vanilla": round(value / v1, 2), "workloads": [cfg.name, van1.name]}}
        if base.batch in blk and base.batch in vtk:
            cmp["decode_heavy"] = {"block": blk[base.batch], "vanilla": vtk[base.batch],
                                   "block_over_vanilla": round(blk[base.batch] / vtk[base.batch], 2),
                                   "workloads": [base.name, van.name]}
        if blk and vtk:
            bb, bv = max(blk), max(vtk)
            cmp["largest_batches_swept"] = {"block_batch": bb, "vanilla_batch": bv,
                                            "block_over_vanilla": round(blk[bb] / vtk[bv], 2)}
        result["vanilla_comparison"] = cmp
        result["batch_sweep"] = {"shape": f"decode-heavy: {base.prompt_len}-token prompts, {base.gen_len} generated; "
                                          "one untimed + one timed generation per point, workspaces sized for the prompt",
                                 "points": pts}
        result["pages_claim"] = PAGES_CLAIM
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(cfg, min(args.cpu_rows, cfg.batch), min(args.cpu_tokens, cfg.gen_len))
    line = json.dumps(result)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
