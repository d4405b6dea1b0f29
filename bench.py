"""Throughput benchmark of Block Transformer batched inference on one MI355X.

One step = one greedy generation over the batch: bt_prefill of the whole prompt, then G-1
bt_decode_step calls (the whole hot path: embedder, block decoder, prefix, token decoder,
classifier).  Inputs are resident in HBM before the timed region starts.  Prints one JSON line.

Workloads (synthetic random-init weights N(0, 0.02^2), uniform random prompt ids):
  c1_prefill_heavy  d=768, 6+6 layers, L_B=4, P=1, V=50304, batch 64, 2048-token prompt, 128 generated
  c2_decode_heavy   same model, batch 256, 128-token prompt, 2048 generated (reported alongside)
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "generated tokens/sec @1 MI355X (prefill- & decode-heavy); decode HBM GB/s"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 / bf16 MFMA, TFLOP/s


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def describe(cfg):
    return (f"{cfg.name}: Block Transformer d={cfg.d_model} {cfg.n_block_layers}+{cfg.n_token_layers} layers "
            f"H={cfg.n_heads}{'' if cfg.kv_heads == cfg.n_heads else f' H_kv={cfg.kv_heads}'} MLP={cfg.d_mlp} "
            f"L_B={cfg.block_len} P={cfg.prefix_len} V={cfg.vocab}"
            f"{'' if cfg.context_mode == 'prefix' else f' context={cfg.context_mode}'}, "
            f"batch {cfg.batch}, {cfg.prompt_len}-token prompt, {cfg.gen_len} generated")


class Runner:
    def __init__(self, cfg, prompt_sized=False):
        """prompt_sized: size the prefill activations for this prompt only (max_prompt_tokens), as a
        server that knows its longest prompt would; the caches are sized for prompt + generation."""
        import torch

        import bt_workloads as wl
        import hierarchical_global_local_amd as hg
        self.torch, self.cfg = torch, cfg
        self.G = cfg.gen_len
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
    return {"kernel_class": "decode/attn_block_decode", "bound": "hbm", "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
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
GEMM_SOURCE = os.path.join(ROOT, "hierarchical_global_local_amd", "csrc", "gemm_decode.hip")


def _rocprof_db(d):
    import glob
    found = glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True)
    if not found:
        raise FileNotFoundError(f"no rocprofv3 results database under {d}")
    return found[0]


def summarize_rocprof(d, top=25):
    """Per-kernel totals of a rocprofv3 --kernel-trace run (the same figures --stats reports)."""
    import sqlite3
    cur = sqlite3.connect(_rocprof_db(d)).cursor()
    rows = list(cur.execute("select name, count(*), sum(end-start), avg(end-start), min(end-start), max(end-start) "
                            "from kernels group by name order by sum(end-start) desc"))
    total = sum(r[2] for r in rows)
    out = [f"{'total_ms':>10} {'pct':>6} {'calls':>7} {'avg_us':>9} {'min_us':>9} {'max_us':>9}  kernel"]
    for name, n, tot, avg, mn, mx in rows[:top]:
        out.append(f"{tot / 1e6:10.3f} {100 * tot / total:6.2f} {n:7d} {avg / 1e3:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f}  {name[:140]}")
    return "\n".join(out)


def _counter_per_dispatch(d, counter):
    import sqlite3
    cur = sqlite3.connect(_rocprof_db(d)).cursor()
    rows = cur.execute("select kernel_name, counter_name, value from counters_collection")
    per = {}
    for kname, cname, value in rows:
        if cname.startswith(counter):
            per.setdefault(kname, []).append(float(value))
    return per


def source_hash(path=GEMM_SOURCE):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_counters(fetch_dir, write_dir, kernel_pattern, kernel_class):
    """Average HBM bytes per dispatch of the kernel matching kernel_pattern (of class kernel_class),
    from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for the 1 GiB reference copy (--copy-calibration).  Written to profiles/ with the hash of the
    decode GEMM source (which holds both decode GEMM kernels and their configuration tables)."""
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
           "kernel_class": kernel_class, "gemm_source_sha256_16": source_hash()}
    os.makedirs(PROFILES, exist_ok=True)
    out_json = traffic_json(kernel_class)
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    # readable summary of the two counter runs next to it
    lines = [f"# HBM traffic of the {kernel_class} kernel ({name[:60]}...) in c1_prefill_heavy",
             "# commands (two passes, one counter each; the 1 GiB reference copy precedes the workload):",
             "#   cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT"]
    for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        lines.append(f"#   rocprofv3 --pmc {c} -d {d} -o run -- python3 bench.py --steps 1 --warmup 0 "
                     "--decode-config none --no-cpu-baseline --no-profile --copy-calibration")
    lines.append(f"#   python bench.py --traffic {fetch_dir} {write_dir} --kernel {kernel_pattern} --kernel-class {kernel_class}")
    lines.append(f"# scaling: FETCH_SIZE of the 1 GiB copy reads {max(copy_f):.0f} KiB (x{f_scale:.3f}), "
                 f"WRITE_SIZE {max(copy_w):.0f} KiB (x{w_scale:.3f})")
    lines.append("# per-kernel averages (KiB per dispatch, unscaled), the 10 most frequent kernels:")
    for cname, d in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        for k, vs in sorted(d.items(), key=lambda kv: -len(kv[1]))[:10]:
            lines.append(f"{cname}  {len(vs):6d}  {sum(vs) / len(vs):10.1f}  {k[:110]}")
    lines.append(f"# result ({os.path.relpath(out_json, ROOT)}): fetch {fb / 1e6:.2f} MB + write {wb / 1e6:.2f} MB "
                 f"per launch = {(fb + wb) / 1e6:.2f} MB")
    with open(os.path.join(PROFILES, "counters_" + kernel_class.replace("/", "_") + "_c1.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return res


def stored_traffic(kernel_class):
    """Counter-measured bytes per launch of a decode kernel class, or None if absent or if the decode
    GEMM source changed since the counters were taken."""
    try:
        with open(traffic_json(kernel_class)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("gemm_source_sha256_16") == source_hash() else None


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
            "host": platform.processor() or platform.machine(), "host_cpus": os.cpu_count()}


def batch_sweep(args):
    """Throughput against batch size at one prompt / generation shape (the pages measure both
    models at their largest batch and report batch sensitivity).  Workspaces are sized for the
    prompt (max_prompt_tokens) so the batch is bounded by the caches; points that do not fit in HBM
    are reported as such."""
    import torch

    import bt_workloads as wl
    base = wl.get_config(args.sweep_config)
    todo = [(base, int(b)) for b in args.batch_sweep.split(",")]
    if args.sweep_vanilla:
        van = wl.get_config({"c2_decode_heavy": "v2_vanilla_decode_heavy",
                             "c1_prefill_heavy": "v1_vanilla_prefill_heavy"}[args.sweep_config])
        todo += [(van, int(b)) for b in args.sweep_vanilla.split(",")]
    rows = []
    for cfg0, B in todo:
        cfg = cfg0.with_(batch=B)
        rec = {"model": cfg0.name, "batch": B}
        try:
            r = Runner(cfg, prompt_sized=True)
            t = r.timed(1, 1)
            rec.update(tokens_per_s=round(B * cfg.gen_len / (t["ms_per_step"] * 1e-3), 1),
                       decode_tokens_per_s=round(B * (cfg.gen_len - 1) / (t["decode_ms"] * 1e-3), 1),
                       ms_per_step=round(t["ms_per_step"], 2), prefill_ms=round(t["prefill_ms"], 2),
                       decode_ms=round(t["decode_ms"], 2),
                       workspace_gib=round(r.model.workspace.numel() / 2 ** 30, 2))
            del r
        except torch.cuda.OutOfMemoryError:
            rec["result"] = "does not fit in HBM"
        torch.cuda.empty_cache()
        log(f"[sweep] {rec}")
        rows.append(rec)
    line = json.dumps({"batch_sweep": describe(base), "gen_len": base.gen_len, "prompt_len": base.prompt_len,
                       "points": rows})
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


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
    ap.add_argument("--kernel", default=None, help="kernel-name pattern for --traffic")
    ap.add_argument("--kernel-class", default="decode/gemm_qkv_up", help="kernel class of --kernel")
    ap.add_argument("--compare-vanilla", action="store_true",
                    help="also time token-level transformers of the same width and depth on the same kernels")
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
    if args.traffic:
        print(json.dumps(traffic_from_counters(args.traffic[0], args.traffic[1], args.kernel, args.kernel_class),
                         indent=1))
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
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t["ms_per_step"], 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "compute": "bf16 weights; matrix operands and KV caches fp16 (exact for bf16 weights after a 2^8 "
                   "pre-scale), fp32 accumulation, softmax, LayerNorm and residual stream",
        "data": "synthetic (random-init N(0,0.02^2) weights, uniform random prompt ids)",
        "config": {"workload": describe(cfg), "global_batch": B, "seq_len": cfg.prompt_len, "gen_len": G},
        "prefill_ms": round(t["prefill_ms"], 3), "decode_ms": round(t["decode_ms"], 3),
        "roofline": None,
    }
    if not args.no_profile:
        prof, prof_ms = r.profiled(args.steps)
        dec_bytes = sum(v["bytes"] for k, v in prof.items() if k.startswith("decode/"))
        pre_flops = sum(v["flops"] for k, v in prof.items() if k.startswith("prefill/"))
        active = {k: v for k, v in prof.items() if v["launches"]}
        dominant = max(active, key=lambda k: active[k]["ms"])
        classes = {k: {"ms_per_step": round(v["ms"], 3), "launches": v["launches"],
                       "rate": roofline_of(k, v)["achieved"], "unit": roofline_of(k, v)["unit"]}
                   for k, v in sorted(active.items(), key=lambda kv: -kv[1]["ms"])}
        for k, v in classes.items():
            log(f"[bench]   {k:28s} {v['ms_per_step']:9.3f} ms/step  {v['launches']:8.1f} launches  {v['rate']:9.1f} {v['unit']}")
        result["prefill_tflops"] = round(pre_flops / (t["prefill_ms"] * 1e-3) / 1e12, 2)
        result["decode_hbm_gbps"] = round(dec_bytes / (t["decode_ms"] * 1e-3) / 1e9, 1)
        result["roofline"] = roofline_of(dominant, prof[dominant])
        result["roofline"]["measured"] = ("HIP events on the library's stream around every launch of the class, "
                                          f"over a profiled repeat of the {args.steps} timed steps")
        if dominant in REPLAYABLE:
            # per-launch events add their own dispatch latency to short kernels: time the same kernel
            # (same shape, weights cycled over the layers) launched back to back instead
            reps = 30 * (cfg.n_token_layers + cfg.n_block_layers)
            us = r.replay_us(REPLAYABLE[dominant], reps)
            roof = result["roofline"]
            roof["event_avg_launch_us_in_steps"] = roof["avg_launch_us"]
            roof["avg_launch_us"] = round(us, 3)
            rate = roof["algorithmic_per_launch"] / (us * 1e-6)
            roof["achieved"] = round(rate / 1e9 if roof["unit"] == "GB/s" else rate / 1e12, 2)
            roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
            roof["measured"] = (f"HIP events on the library's stream around {reps} back-to-back launches of the "
                                f"class's kernel at the decode shape (bt_test_replay, weights cycled over all "
                                f"layers of both decoders), after the timed steps; algorithmic bytes per launch from the profiled "
                                f"repeat of the timed steps")
        tr = stored_traffic(dominant)
        if tr is not None:
            result["roofline"]["traffic"] = round(tr["traffic_bytes_per_launch"], 1)
            result["roofline"]["traffic_source"] = (os.path.relpath(traffic_json(dominant), ROOT) +
                                                    " (FETCH_SIZE + WRITE_SIZE)")
        result["profiled_ms_per_step"] = round(prof_ms, 3)
        result["kernel_classes"] = classes
    del r
    torch.cuda.empty_cache()
    if args.decode_config != "none":
        c2 = wl.get_config(args.decode_config)
        log(f"[bench] {describe(c2)}")
        r2 = Runner(c2)
        t2 = r2.timed(1, 1)
        prof2, _ = r2.profiled(1)
        d_bytes = sum(v["bytes"] for k, v in prof2.items() if k.startswith("decode/"))
        att = prof2["decode/attn_block_decode"]
        dom2 = max((k for k in prof2 if prof2[k]["launches"]), key=lambda k: prof2[k]["ms"])
        result["decode_heavy"] = {
            "workload": describe(c2), "value": round(c2.batch * c2.gen_len / (t2["ms_per_step"] * 1e-3), 1),
            "unit": "tokens/s", "ms_per_step": round(t2["ms_per_step"], 3),
            "prefill_ms": round(t2["prefill_ms"], 3), "decode_ms": round(t2["decode_ms"], 3),
            "decode_tokens_per_s": round(c2.batch * (c2.gen_len - 1) / (t2["decode_ms"] * 1e-3), 1),
            "decode_hbm_gbps": round(d_bytes / (t2["decode_ms"] * 1e-3) / 1e9, 1),
            "block_attn_decode": attn_replay_roofline(r2, c2),
            "dominant": roofline_of(dom2, prof2[dom2]),
        }
        log(f"[bench] decode-heavy: {result['decode_heavy']['value']:.0f} tokens/s, "
            f"decode {result['decode_heavy']['decode_hbm_gbps']} GB/s")
        del r2
        torch.cuda.empty_cache()
    if args.compare_vanilla:
        cmp = {}
        for block_name, van_name in (("c1_prefill_heavy", "v1_vanilla_prefill_heavy"),
                                     ("c2_decode_heavy", "v2_vanilla_decode_heavy")):
            row = {}
            for name in (block_name, van_name):
                c = wl.get_config(name)
                rr = Runner(c)
                tt = rr.timed(1, 1)
                row[name] = {"tokens_per_s": round(c.batch * c.gen_len / (tt["ms_per_step"] * 1e-3), 1),
                             "prefill_ms": round(tt["prefill_ms"], 3), "decode_ms": round(tt["decode_ms"], 3)}
                log(f"[bench] {name}: {row[name]}")
                del rr
                torch.cuda.empty_cache()
            row["block_over_vanilla"] = round(row[block_name]["tokens_per_s"] / row[van_name]["tokens_per_s"], 2)
            cmp[block_name] = row
        result["vanilla_comparison"] = cmp
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
