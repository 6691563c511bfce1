"""Decode-step benchmark of the gfx950 megakernel (one JSON line on stdout).

Workload: the Llama-3.2-1B-shaped decoder (16 layers, hidden 2048, 32 q / 8 kv
heads of 64, SwiGLU 8192, vocab 128256, tied embeddings, bf16 random-init
weights N(0, 0.02), RoPE theta 500000), batch 1, a 496-position context, greedy
decoding.  Weights, tokens and the cached context are seeded synthetic inputs
(the context's K/V are drawn at the scale of a random-init projection instead
of a 496-token prefill); everything is resident in HBM before timing starts.

A step is one decode step of the whole model, one megakernel launch; tokens
chain on the device from step to step.  After W warmup steps, K steps are
timed between a synchronize on each side (`value`); each launch is also
bracketed by HIP events on the stream it runs on.  The same K steps are then
repeated R-1 more times from the same starting state (sequence lengths and
tokens reset, the same K/V positions rewritten), so the per-launch latency
distribution has R*K samples.  The per-operator hipGraph baseline runs the same
blocks; at batch 1 the same K steps also run in one persistent session (the
grid kept resident, steps rung from the host) under "persistent"; the ablations (Table I features switched off one at a time) run one
block each, and the CPU oracle is timed on a bounded sample of the same
workload.  A second workload, batch 32 with per-sequence contexts drawn from
U{256..1024} (the matrix-core path), is reported under "batch32"; the time
to first token of 496-token prompts at batch 16 (the prefill: one megakernel,
two co-resident megakernels, the per-operator graph) under "ttft".

    python bench.py [--steps 64] [--warmup 3] [--reps 5] [--no-cpu] [--no-baseline]
                    [--no-batch32] [--no-ablations] [--no-persistent] [--no-ttft] [--ttft-runs 10]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode step latency (µs) + achieved HBM GB/s, Llama-1B-shape, batch 1 and 32"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CONTEXT = 496
TTFT_PROMPT = 496


def step_bytes(cfg, batch: int, positions_before: np.ndarray) -> float:
    """Algorithmic HBM bytes of one step: every weight once, the cached K/V of
    each sequence read once (positions 0..p, p the position appended), the new
    K/V written, one embedding row per sequence read, fp32 logits written."""
    w = cfg.weight_bytes()
    kv_per_pos = cfg.n_layers * cfg.n_kv_heads * cfg.head_dim * 2 * cfg.elt_bytes
    n = positions_before.astype(np.float64) + 1.0
    return w + float(np.sum(n * kv_per_pos + kv_per_pos + cfg.hidden * cfg.elt_bytes + cfg.vocab * 4))


def profile_record(name: str, shash: str):
    """A recorded profile summary (profiles/<name>), if it was taken on the
    current sources."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    return t if t.get("source_hash") == shash else None


def tile_read_ceiling():
    """The repository's measured streaming ceiling: the best tile-read
    bandwidth of the microbenchmark (64 KiB tiles into registers, the
    megakernel's load shape), from its recorded output."""
    path = os.path.join(ROOT, "profiles", "microbench_gfx950.md")
    best = None
    if os.path.exists(path):
        for line in open(path):
            line = line.strip()
            if line.startswith('{"bench": "tile_read", "mode": 0,'):
                best = max(best or 0.0, json.loads(line)["GBps"])
    return best


def lat(per):
    return {"mean": round(float(per.mean()), 2), "p50": round(float(np.percentile(per, 50)), 2),
            "p95": round(float(np.percentile(per, 95)), 2), "p99": round(float(np.percentile(per, 99)), 2),
            "min": round(float(per.min()), 2), "samples": int(per.size)}


class Workload:
    """Device state of one workload: KV cache, lengths, tokens, logits."""

    def __init__(self, wpk, torch, cfg, batch, lens0, tok0, cap, dev):
        import synth
        self.wpk, self.torch, self.cfg, self.batch, self.dev = wpk, torch, cfg, batch, dev
        self.lens0, self.tok0, self.cap = lens0, tok0, cap
        kc_np, vc_np = synth.synthetic_kv(cfg, batch, cap, lens0)
        self.kc = torch.from_numpy(kc_np.view(np.int16)).to(dev)
        self.vc = torch.from_numpy(vc_np.view(np.int16)).to(dev)
        self.seq = torch.from_numpy(lens0.copy()).to(dev)
        self.tokens = torch.from_numpy(tok0.copy()).to(dev)
        self.logits = torch.empty((batch, cfg.vocab), dtype=torch.float32, device=dev)
        self.kv = wpk.wpk_kv(self.kc.data_ptr(), self.vc.data_ptr(), self.seq.data_ptr())
        self.stream = torch.cuda.current_stream(dev)

    def reset(self):
        self.seq.copy_(self.torch.from_numpy(self.lens0))
        self.tokens.copy_(self.torch.from_numpy(self.tok0))
        self.torch.cuda.synchronize(self.dev)

    def step(self, plan):
        self.wpk.check(self.wpk.wpk_step(plan, self.tokens.data_ptr(), self.kv, self.logits.data_ptr(),
                                         self.stream.cuda_stream), plan, "wpk_step")

    def block(self, plan, warmup, steps, label):
        """Warmup, then `steps` launches each bracketed by HIP events on the
        launch stream, between synchronizes.  Returns (wall seconds, per-launch
        µs, algorithmic bytes per launch)."""
        torch, wpk = self.torch, self.wpk
        self.reset()
        for _ in range(warmup):
            self.step(plan)
        wpk.check(wpk.wpk_sync(plan), plan, label)
        positions = self.seq.cpu().numpy().astype(np.int64)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize(self.dev)
        w0 = time.perf_counter()
        for e0, e1 in ev:
            e0.record(self.stream)
            self.step(plan)
            e1.record(self.stream)
        torch.cuda.synchronize(self.dev)
        wall = time.perf_counter() - w0
        wpk.check(wpk.wpk_sync(plan), plan, label)
        per = np.array([a.elapsed_time(b) * 1000.0 for a, b in ev])
        byts = np.array([step_bytes(self.cfg, self.batch, positions + i) for i in range(steps)])
        return wall, per, byts


def progress(msg: str) -> None:
    """A progress line on stderr (the JSON line stays alone on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measure(wpk, W: Workload, desc, args, baseline: bool, ablations):
    """The timed block (value), R-1 repeated blocks for the latency
    distribution, the graph baseline's blocks and one block per ablation."""
    plan = wpk.wpk_build(desc.desc, W.batch, W.cap)
    if not plan:
        raise RuntimeError("wpk_build: " + wpk.wpk_last_error(None))
    info = wpk.wpk_get_info(plan)
    blocks = [W.block(plan, args.warmup, args.steps, "megakernel") for _ in range(args.reps)]
    progress(f"batch {W.batch}: megakernel, {args.reps} x {args.steps} steps")
    wpk.wpk_destroy(plan)
    out = {"wall": blocks[0][0], "per": np.concatenate([b[1] for b in blocks]), "bytes": blocks[0][2],
           "block_us": [round(b[0] / args.steps * 1e6, 2) for b in blocks], "info": info}
    if baseline:
        bplan = wpk.wpk_build_graph_baseline(desc.desc, W.batch, W.cap)
        if not bplan:
            raise RuntimeError("baseline build: " + wpk.wpk_last_error(None))
        bb = [W.block(bplan, args.warmup, args.steps, "graph baseline") for _ in range(args.reps)]
        progress(f"batch {W.batch}: graph baseline")
        wpk.wpk_destroy(bplan)
        bper = np.concatenate([b[1] for b in bb])
        out["baseline"] = {"value": round(bb[0][0] / args.steps * 1e6, 2), "unit": "µs/step",
                           "latency_us": lat(bper),
                           "megakernel_speedup": round(float(bper.mean() / out["per"].mean()), 3)}
    if W.batch <= 4 and not args.no_persistent:
        out["persistent"] = persistent_block(wpk, W, desc, args, out["per"])
        progress(f"batch {W.batch}: persistent session")
    res = {}
    for name, opts, option in ablations:
        p = wpk.wpk_build_ex(desc.desc, W.batch, W.cap, opts)
        if not p:
            res[name] = {"error": wpk.wpk_last_error(None)}
            continue
        if option:
            wpk.check(wpk.wpk_set_option(p, option[0], option[1]), p, name)
        wall, per, _ = W.block(p, args.warmup, args.steps, name)
        wpk.wpk_destroy(p)
        progress(f"batch {W.batch}: ablation {name}")
        res[name] = {"value": round(wall / args.steps * 1e6, 2), "unit": "µs/step",
                     "latency_mean_us": round(float(per.mean()), 2),
                     "vs_default": round(float(per.mean() / out["per"].mean()), 3)}
    if res:
        out["ablations"] = res
    return out


def persistent_block(wpk, W: Workload, desc, args, launched_per):
    """The same K steps run by one resident grid (a persistent session): the
    host rings all K at once after W warmup steps and waits for the count of
    finished steps in pinned host memory; the device stamps each step (grant
    seen, last worker out)."""
    plan = wpk.wpk_build(desc.desc, W.batch, W.cap)
    if not plan:
        raise RuntimeError("wpk_build: " + wpk.wpk_last_error(None))
    W.reset()
    wpk.check(wpk.wpk_persist_begin(plan, W.tokens.data_ptr(), W.kv, W.logits.data_ptr(), W.stream.cuda_stream),
              plan, "persist begin")
    wpk.check(wpk.wpk_persist_ring(plan, args.warmup), plan, "ring")
    wpk.check(wpk.wpk_persist_wait(plan, args.warmup, 60_000_000), plan, "wait")
    t0 = time.perf_counter()
    wpk.check(wpk.wpk_persist_ring(plan, args.steps), plan, "ring")
    wpk.check(wpk.wpk_persist_wait(plan, args.warmup + args.steps, 60_000_000), plan, "wait")
    wall = time.perf_counter() - t0
    wpk.check(wpk.wpk_persist_end(plan), plan, "persist end")
    rc, t = wpk.wpk_persist_times(plan, args.warmup + args.steps)
    wpk.check(rc, plan, "persist times")
    wpk.wpk_destroy(plan)
    t = t[args.warmup:].astype(np.float64) / 100.0  # s_memrealtime ticks (100 MHz) -> µs
    dev = t[:, 1] - t[:, 0]
    gaps = t[1:, 0] - t[:-1, 1]
    return {"value": round(wall / args.steps * 1e6, 2), "unit": "µs/step",
            "device_step_us": lat(dev), "step_boundary_us": lat(gaps) if gaps.size else None,
            "vs_launched_event_mean": round(float(launched_per.mean() / (wall / args.steps * 1e6)), 3),
            "how": "one cooperative grid for all steps; K steps rung at once; host waits on pinned memory"}


def ttft_block(wpk, torch, cfg, desc, args, dev):
    """Time to first token (the Table III workload of "One Megakernel is Not
    Enough" at the Llama-3.2-1B shape): batch 16, a 496-token prompt of
    seeded random ids, prefill through every layer and the LM head on each
    sequence's last prompt row (the first greedy token).  Run as one
    megakernel, as two co-resident megakernels (attention tiles in their own
    worker pool of 32, 64 or 128 of the 256 workers) and as the per-operator
    hipGraph; each run is bracketed by HIP events on the launch stream."""
    import synth
    batch, P, cap = 16, TTFT_PROMPT, 512
    prompt = torch.from_numpy(synth.prompt_tokens(cfg, batch, P, seed=4).astype(np.int32)).to(dev)
    shape = (cfg.n_layers, batch, cfg.n_kv_heads, cap, cfg.head_dim)
    kc = torch.zeros(shape, dtype=torch.int16, device=dev)
    vc = torch.zeros(shape, dtype=torch.int16, device=dev)
    seq = torch.zeros(batch, dtype=torch.int32, device=dev)
    logits = torch.empty((batch, cfg.vocab), dtype=torch.float32, device=dev)
    tok = torch.empty(batch, dtype=torch.int32, device=dev)
    kv = wpk.wpk_kv(kc.data_ptr(), vc.data_ptr(), seq.data_ptr())
    stream = torch.cuda.current_stream(dev)
    out = {"workload": f"Llama-3.2-1B-shape prefill, batch {batch}, {P}-token prompts, first greedy token",
           "batch": batch, "prompt": P}
    first = None
    for name, mode, w1 in (("megakernel", wpk.WPK_PREFILL_MEGAKERNEL, 0), ("split_32", wpk.WPK_PREFILL_SPLIT, 32),
                           ("split_64", wpk.WPK_PREFILL_SPLIT, 64), ("split_128", wpk.WPK_PREFILL_SPLIT, 128),
                           ("graph_baseline", wpk.WPK_PREFILL_GRAPH, 0)):
        plan = wpk.wpk_build_prefill(desc.desc, batch, cap, P, wpk.wpk_prefill_opts(mode=mode, split_workers=w1))
        if not plan:
            raise RuntimeError("wpk_build_prefill: " + wpk.wpk_prefill_last_error(None))
        info = wpk.wpk_prefill_get_info(plan)

        def go():
            wpk.check_prefill(wpk.wpk_prefill(plan, prompt.data_ptr(), kv, logits.data_ptr(), tok.data_ptr(),
                                              stream.cuda_stream), plan, name)
        for _ in range(args.warmup):
            go()
        wpk.check_prefill(wpk.wpk_prefill_sync(plan), plan, name)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.ttft_runs)]
        torch.cuda.synchronize(dev)
        w0 = time.perf_counter()
        for e0, e1 in ev:
            e0.record(stream)
            go()
            e1.record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - w0
        wpk.check_prefill(wpk.wpk_prefill_sync(plan), plan, name)
        per = np.array([a.elapsed_time(b) * 1000.0 for a, b in ev])
        toks = tok.cpu().numpy().tolist()
        if first is None:
            first = toks
        wpk.wpk_prefill_destroy(plan)
        progress(f"ttft: {name}")
        out[name] = {"value": round(wall / args.ttft_runs * 1e6, 1), "unit": "µs", "latency_us": lat(per),
                     "workers": info.workers, "split_workers": info.split_workers, "tiles": info.n_tiles,
                     "kernels": 1 if mode != wpk.WPK_PREFILL_GRAPH else info.n_phases,
                     "same_tokens_as_megakernel": toks == first}
        out["flops"] = info.flops
    mk = out["megakernel"]["latency_us"]["mean"]
    achieved = out["flops"] / (mk * 1e-6) / 1e12
    out["mfma"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                   "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                   "kernel": "wpk::prefill_megakernel", "source_hash": wpk.prefill_source_hash()}
    best = min(("split_32", "split_64", "split_128"), key=lambda k: out[k]["latency_us"]["mean"])
    out["best_split"] = best
    out["split_vs_megakernel"] = round(out[best]["latency_us"]["mean"] / mk, 3)
    out["graph_vs_megakernel"] = round(out["graph_baseline"]["latency_us"]["mean"] / mk, 3)
    out["first_tokens"] = first
    return out


def roofline(byts, per, shash, kernel_key, traffic_name):
    achieved = float(np.mean(byts) / (per.mean() * 1e-6) / 1e9)
    traffic = profile_record(traffic_name, shash)
    kd = profile_record("megakernel_kernel_durations.json", shash)
    rk = kd.get(kernel_key) if kd else None
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic.get("hbm_bytes_per_launch") if traffic else None,
            "bytes_per_launch": round(float(np.mean(byts))),
            "kernel": "wpk::megakernel", "kernel_us_events": round(float(per.mean()), 2),
            "kernel_us_rocprof": rk["average_us"] if rk else None,
            "tile_read_ceiling_GBps": tile_read_ceiling(), "source_hash": shash}


def run(args):
    import torch

    import persistent_megakernel_latency_amd as wpk
    import synth

    cfg = synth.LLAMA_1B
    torch.cuda.init()
    dev = torch.device("cuda", 0)
    t0 = time.time()
    weights = synth.make_weights(cfg)
    desc, tensors = wpk.model_from_weights(cfg, weights, dev)
    batch = 1
    lens0 = np.full(batch, CONTEXT, np.int32)
    tok0 = synth.prompt_tokens(cfg, batch, CONTEXT)[:, -1].astype(np.int32)
    cap = int(np.ceil((CONTEXT + args.warmup + args.steps + 2) / 64.0) * 64)
    W1 = Workload(wpk, torch, cfg, batch, lens0, tok0, cap, dev)
    setup_s = time.time() - t0
    ab1 = [] if args.no_ablations else [
        ("weight_prefetch_off", None, (wpk.WPK_OPT_PREFETCH, 0)),
        ("barrier_edges", wpk.wpk_build_opts(barrier_edges=1), None),
        ("cooperative_launch", None, (wpk.WPK_OPT_LAUNCH, 1)),
        ("co_resident_split_attention_128", wpk.wpk_build_opts(split_workers=128), None),
    ]
    m = measure(wpk, W1, desc, args, not args.no_baseline, ab1)
    wall, per, byts, info = m["wall"], m["per"], m["bytes"], m["info"]
    shash = wpk.source_hash()
    result = {
        "metric": METRIC,
        "value": round(wall / args.steps * 1e6, 2),
        "unit": "µs/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"Llama-3.2-1B-shape decode step, batch {batch}, context {CONTEXT}, greedy",
                   "batch": batch, "context": CONTEXT, "layers": cfg.n_layers, "hidden": cfg.hidden,
                   "q_heads": cfg.n_q_heads, "kv_heads": cfg.n_kv_heads, "ffn": cfg.ffn, "vocab": cfg.vocab,
                   "workers": info.workers, "tiles_per_step": info.n_tiles},
        "repetitions": {"reps": args.reps, "block_us_per_step": m["block_us"]},
        "latency_us": lat(per),
        "tokens_per_s": round(batch * args.steps / wall, 1),
    }
    rl = roofline(byts, per, shash, "batch1", "megakernel_llama1b_b1_traffic.json")
    result["hbm_GBps"] = rl["achieved"]
    result["roofline"] = rl
    if "baseline" in m:
        result["graph_baseline"] = m["baseline"]
    if "persistent" in m:
        result["persistent"] = m["persistent"]
    if "ablations" in m:
        result["ablations"] = m["ablations"]
    del W1

    if not args.no_batch32:
        b32 = 32
        lens32 = synth.context_lengths(b32)
        tok32 = synth.prompt_tokens(cfg, b32, 1)[:, 0].astype(np.int32)
        cap32 = int(np.ceil((int(lens32.max()) + args.warmup + args.steps + 2) / 64.0) * 64)
        W32 = Workload(wpk, torch, cfg, b32, lens32, tok32, cap32, dev)
        ab32 = [] if args.no_ablations else [
            ("lds_forwarding_chained_attention", wpk.wpk_build_opts(forward=1), None),
            ("barrier_edges", wpk.wpk_build_opts(barrier_edges=1), None),
            ("weight_prefetch_off", None, (wpk.WPK_OPT_PREFETCH, 0)),
            ("co_resident_split_attention_128", wpk.wpk_build_opts(split_workers=128), None),
            ("co_resident_split_attention_256", wpk.wpk_build_opts(split_workers=256), None),
        ]
        m32 = measure(wpk, W32, desc, args, not args.no_baseline, ab32)
        w32, per32, by32 = m32["wall"], m32["per"], m32["bytes"]
        flops = 2.0 * cfg.n_matrix_params() * b32  # projections, MLP and LM head
        rl32 = roofline(by32, per32, shash, "batch32", "megakernel_llama1b_b32_traffic.json")
        result["batch32"] = {
            "workload": "Llama-3.2-1B-shape decode step, batch 32, contexts U{256..1024}, greedy",
            "value": round(w32 / args.steps * 1e6, 2), "unit": "µs/step", "latency_us": lat(per32),
            "repetitions": {"reps": args.reps, "block_us_per_step": m32["block_us"]},
            "tokens_per_s": round(b32 * args.steps / w32, 1), "hbm_GBps": rl32["achieved"],
            "roofline": rl32,
            "mfma": {"flops_per_step": flops, "achieved_TFLOPs": round(flops / (per32.mean() * 1e-6) / 1e12, 2),
                     "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                     "frac": round(flops / (per32.mean() * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4)},
            "workers": m32["info"].workers, "tiles_per_step": m32["info"].n_tiles}
        if "baseline" in m32:
            result["batch32"]["graph_baseline"] = m32["baseline"]
        if "ablations" in m32:
            result["batch32"]["ablations"] = m32["ablations"]
        del W32

    if not args.no_ttft:
        result["ttft"] = ttft_block(wpk, torch, cfg, desc, args, dev)

    if not args.no_cpu:
        progress("cpu baseline (oracle)")
        kc_np, vc_np = synth.synthetic_kv(cfg, batch, cap, lens0)
        result["cpu_baseline"] = cpu_baseline(cfg, weights, batch, kc_np, vc_np, lens0, tok0, args.cpu_seconds)
    result["setup_s"] = round(setup_s, 1)
    return result


def cpu_baseline(cfg, weights, batch, kc_np, vc_np, lens0, tok0, budget_s):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    same workload: consecutive decode steps from the same context until
    about `budget_s` seconds have passed (at least two)."""
    import oracle

    model = oracle.Model(cfg, weights)
    kc, vc, sl, tok = kc_np.copy(), vc_np.copy(), lens0.copy(), tok0.copy()
    times = []
    t_all = time.perf_counter()
    while len(times) < 2 or (time.perf_counter() - t_all < budget_s and len(times) < 64):
        t = time.perf_counter()
        _, tok = model.step(tok, kc, vc, sl)
        times.append(time.perf_counter() - t)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(float(np.mean(times)) * 1e6, 1), "unit": "µs/step", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(times)} consecutive float64 decode steps of the same model, batch {batch}, "
                      f"from the same {CONTEXT}-position context"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-baseline", action="store_true")
    ap.add_argument("--no-batch32", action="store_true")
    ap.add_argument("--no-ablations", action="store_true")
    ap.add_argument("--no-persistent", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-ttft", action="store_true")
    ap.add_argument("--ttft-runs", type=int, default=10)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this build runs on a "
              "single GPU (batched sequences would shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)
    if args.reps < 1 or args.steps < 1:
        print("--reps and --steps must be positive", file=sys.stderr)
        sys.exit(2)
    print(json.dumps(run(args)))


if __name__ == "__main__":
    main()
