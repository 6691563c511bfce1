"""Decode-step benchmark of the gfx950 megakernel (one JSON line on stdout).

Workload: the Llama-3.2-1B-shaped decoder (16 layers, hidden 2048, 32 q / 8 kv
heads of 64, SwiGLU 8192, vocab 128256, tied embeddings, bf16 random-init
weights N(0, 0.02), RoPE theta 500000), batch 1, a 496-position context, greedy
decoding.  Weights, tokens and the cached context are seeded synthetic inputs
(the context's K/V are drawn at the scale of a random-init projection instead
of a 496-token prefill); everything is resident in HBM before timing starts.

A step is one decode step of the whole model, one megakernel launch; tokens
chain on the device from step to step.  K steps are timed between a
synchronize on each side; each launch is also bracketed by HIP events on the
stream it runs on, which gives the per-step latency distribution and the
kernel duration used for the roofline.  The same K steps are then run through
the per-operator hipGraph baseline, and the CPU oracle is timed on a bounded
sample of the same workload.  A second workload, batch 32 with per-sequence
contexts drawn from U{256..1024} (the matrix-core path), is reported in the
same line under "batch32", with its own graph baseline.

    python bench.py [--steps 64] [--warmup 3] [--batch 1] [--no-cpu] [--no-baseline] [--no-batch32]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode step latency (µs) + achieved HBM GB/s, Llama-1B-shape, batch 1 and 32"
HBM_PEAK_GBPS = 8000.0
CONTEXT = 496


def source_hash() -> str:
    h = hashlib.sha256()
    for f in ("megakernel.hip", "plan.h"):
        with open(os.path.join(ROOT, "persistent_megakernel_latency_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def step_bytes(cfg, batch: int, positions_before: np.ndarray) -> float:
    """Algorithmic HBM bytes of one step: every weight once, the cached K/V of
    each sequence read once (positions 0..p, p the position appended), the new
    K/V written, one embedding row per sequence read, fp32 logits written."""
    w = cfg.weight_bytes()
    kv_per_pos = cfg.n_layers * cfg.n_kv_heads * cfg.head_dim * 2 * cfg.elt_bytes
    n = positions_before.astype(np.float64) + 1.0
    return w + float(np.sum(n * kv_per_pos + kv_per_pos + cfg.hidden * cfg.elt_bytes + cfg.vocab * 4))


def traffic_from_profile(shash: str, per_launch_bytes: float, name: str = "megakernel_llama1b_b1_traffic.json"):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != shash:
        return None  # the kernel changed since the counters were taken
    return t.get("hbm_bytes_per_launch")


def measure(wpk, torch, cfg, desc, batch, lens0, tok0, args, dev, baseline: bool):
    """Times K decode steps of one workload on the megakernel (and, if asked,
    on the per-operator graph baseline) from the same starting state."""
    cap = int(np.ceil((int(lens0.max()) + args.warmup + args.steps + 2) / 64.0) * 64)
    kc_np, vc_np = synth_kv(cfg, batch, cap, lens0)
    kc = torch.from_numpy(kc_np.view(np.int16)).to(dev)
    vc = torch.from_numpy(vc_np.view(np.int16)).to(dev)
    seq = torch.from_numpy(lens0.copy()).to(dev)
    tokens = torch.from_numpy(tok0.copy()).to(dev)
    logits = torch.empty((batch, cfg.vocab), dtype=torch.float32, device=dev)
    kv = wpk.wpk_kv(kc.data_ptr(), vc.data_ptr(), seq.data_ptr())
    stream = torch.cuda.current_stream(dev)

    def reset_state():
        seq.copy_(torch.from_numpy(lens0))
        tokens.copy_(torch.from_numpy(tok0))
        torch.cuda.synchronize(dev)

    def timed(plan, label):
        reset_state()
        for _ in range(args.warmup):
            wpk.check(wpk.wpk_step(plan, tokens.data_ptr(), kv, logits.data_ptr(), stream.cuda_stream), plan)
        wpk.check(wpk.wpk_sync(plan), plan, label)
        positions = seq.cpu().numpy().astype(np.int64)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize(dev)
        w0 = time.perf_counter()
        for e0, e1 in ev:
            e0.record(stream)
            wpk.check(wpk.wpk_step(plan, tokens.data_ptr(), kv, logits.data_ptr(), stream.cuda_stream), plan)
            e1.record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - w0
        wpk.check(wpk.wpk_sync(plan), plan, label)
        per = np.array([a.elapsed_time(b) * 1000.0 for a, b in ev])  # microseconds per launch
        byts = np.array([step_bytes(cfg, batch, positions + i) for i in range(args.steps)])
        return wall, per, byts

    plan = wpk.wpk_build(desc.desc, batch, cap)
    if not plan:
        raise RuntimeError("wpk_build: " + wpk.wpk_last_error(None))
    info = wpk.wpk_get_info(plan)
    wall, per, byts = timed(plan, "megakernel")
    wpk.wpk_destroy(plan)
    out = {"wall": wall, "per": per, "bytes": byts, "info": info, "kv": (kc_np, vc_np)}
    if baseline:
        bplan = wpk.wpk_build_graph_baseline(desc.desc, batch, cap)
        if not bplan:
            raise RuntimeError("baseline build: " + wpk.wpk_last_error(None))
        bwall, bper, _ = timed(bplan, "graph baseline")
        wpk.wpk_destroy(bplan)
        out["baseline"] = {"value": round(bwall / args.steps * 1e6, 2), "unit": "µs/step",
                           "latency_us": {"mean": round(float(bper.mean()), 2),
                                          "p50": round(float(np.percentile(bper, 50)), 2),
                                          "p95": round(float(np.percentile(bper, 95)), 2)},
                           "megakernel_speedup": round(float(bper.mean() / per.mean()), 3)}
    return out


def synth_kv(cfg, batch, cap, lens):
    import synth

    return synth.synthetic_kv(cfg, batch, cap, lens)


def lat(per):
    return {"mean": round(float(per.mean()), 2), "p50": round(float(np.percentile(per, 50)), 2),
            "p95": round(float(np.percentile(per, 95)), 2), "p99": round(float(np.percentile(per, 99)), 2),
            "min": round(float(per.min()), 2)}


def run(args):
    import torch

    import persistent_megakernel_latency_amd as wpk
    import synth

    cfg = synth.LLAMA_1B
    batch = args.batch
    torch.cuda.init()
    dev = torch.device("cuda", 0)
    t0 = time.time()
    weights = synth.make_weights(cfg)
    desc, tensors = wpk.model_from_weights(cfg, weights, dev)
    lens0 = np.full(batch, CONTEXT, np.int32)
    tok0 = synth.prompt_tokens(cfg, batch, CONTEXT)[:, -1].astype(np.int32)
    setup_s = time.time() - t0
    m = measure(wpk, torch, cfg, desc, batch, lens0, tok0, args, dev, not args.no_baseline)
    wall, per, byts, info = m["wall"], m["per"], m["bytes"], m["info"]

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
        "latency_us": lat(per),
        "tokens_per_s": round(batch * args.steps / wall, 1),
    }
    achieved = float(np.mean(byts) / (per.mean() * 1e-6) / 1e9)
    shash = source_hash()
    traffic = traffic_from_profile(shash, float(np.mean(byts)))
    result["hbm_GBps"] = round(achieved, 1)
    result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                          "bytes_per_launch": round(float(np.mean(byts))), "kernel": "wpk::megakernel",
                          "kernel_us": round(float(per.mean()), 2), "source_hash": shash}
    if "baseline" in m:
        result["graph_baseline"] = m["baseline"]

    if not args.no_batch32:
        # the batch-32 workload: contexts U{256..1024}, matrix-core projections
        b32 = 32
        lens32 = synth.context_lengths(b32)
        tok32 = synth.prompt_tokens(cfg, b32, 1)[:, 0].astype(np.int32)
        m32 = measure(wpk, torch, cfg, desc, b32, lens32, tok32, args, dev, not args.no_baseline)
        w32, per32, by32 = m32["wall"], m32["per"], m32["bytes"]
        gb = float(np.mean(by32) / (per32.mean() * 1e-6) / 1e9)
        flops = 2.0 * cfg.n_matrix_params() * b32  # projections, MLP and LM head
        result["batch32"] = {
            "workload": "Llama-3.2-1B-shape decode step, batch 32, contexts U{256..1024}, greedy",
            "value": round(w32 / args.steps * 1e6, 2), "unit": "µs/step", "latency_us": lat(per32),
            "tokens_per_s": round(b32 * args.steps / w32, 1), "hbm_GBps": round(gb, 1),
            "roofline": {"bound": "hbm", "achieved": round(gb, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gb / HBM_PEAK_GBPS, 4),
                         "traffic": traffic_from_profile(shash, float(np.mean(by32)),
                                                         "megakernel_llama1b_b32_traffic.json"),
                         "bytes_per_launch": round(float(np.mean(by32))), "kernel_us": round(float(per32.mean()), 2)},
            "mfma": {"flops_per_step": flops, "achieved_TFLOPs": round(flops / (per32.mean() * 1e-6) / 1e12, 2),
                     "peak_TFLOPs": 2500.0,
                     "frac": round(flops / (per32.mean() * 1e-6) / 2.5e15, 4)},
            "workers": m32["info"].workers, "tiles_per_step": m32["info"].n_tiles}
        if "baseline" in m32:
            result["batch32"]["graph_baseline"] = m32["baseline"]

    if not args.no_cpu:
        kc_np, vc_np = m["kv"]
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
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-baseline", action="store_true")
    ap.add_argument("--no-batch32", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this build runs on a "
              "single GPU (batched sequences would shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)
    print(json.dumps(run(args)))


if __name__ == "__main__":
    main()
