"""The planner for the prompt prefill (time to first token): per-operator
profiles in, each candidate design's prefill simulated on its own tile DAG,
the best design out -- the method of "One Megakernel is Not Enough" (the
abstract and Table I) applied to the prefill workload of its Table III
Llama 3.2 1B row.

Candidate designs: one megakernel, two co-resident megakernels with the
attention tiles in a pool of 32, 64 or 128 of the workers, and the
conventional one kernel per (layer, operator) in a hipGraph.

Profiles (GPU): one logged megakernel prefill of the workload; each tile
type's cost is the median duration of its tiles, attention tiles' cost a
fixed part plus one per 32-key step of their causal span (a least-squares
fit over the layer's tiles), and the hop is the median delay between a
group's last publish and a waiting tile's start.  The same run also times
every design (HIP events), which is what the predictions are checked
against.

    python -m persistent_megakernel_latency_amd.prefill_planner measure --out profiles/prefill_planner_profile.json
    python -m persistent_megakernel_latency_amd.prefill_planner validate profiles/prefill_planner_profile.json \\
        [--markdown profiles/prefill_planner_validation.md]
"""
from __future__ import annotations

import argparse
import itertools
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

DESIGNS = ("megakernel", "split_32", "split_64", "split_128", "conventional")
LAUNCH_GAP_US = 2.0  # between two graph-replayed kernels (the decode baseline's fit is of this order)


def design_opts(wpk, name):
    if name == "megakernel":
        return wpk.wpk_prefill_opts(mode=wpk.WPK_PREFILL_MEGAKERNEL)
    if name.startswith("split_"):
        return wpk.wpk_prefill_opts(mode=wpk.WPK_PREFILL_SPLIT, split_workers=int(name.split("_")[1]))
    return wpk.wpk_prefill_opts(mode=wpk.WPK_PREFILL_GRAPH)


def costs_from_log(log, ty, wait, signal, steps):
    """Per-type median tile time (µs), the attention step cost, and the hop."""
    tick = 0.01  # s_memrealtime: 100 MHz
    st = log["t_start"].astype(np.float64) * tick
    en = log["t_end"].astype(np.float64) * tick
    dur = en - st
    tile_us = {}
    for t in sorted(set(ty.tolist())):
        tile_us[int(t)] = float(np.median(dur[ty == t]))
    att = ty == 3
    step_us = 0.0
    if att.any():
        x = steps[att].astype(np.float64)
        A = np.stack([np.ones_like(x), x], 1)
        (a, b), *_ = np.linalg.lstsq(A, dur[att], rcond=None)
        tile_us[3], step_us = float(max(a, 0.0)), float(max(b, 0.0))
    # hop: a waiting tile's start minus its group's last publish, where it waited
    last = {}
    for i in np.nonzero(signal >= 0)[0]:
        g = int(signal[i])
        last[g] = max(last.get(g, -1e300), en[i])
    d = np.array([st[i] - last[int(wait[i])] for i in np.nonzero(wait >= 0)[0] if int(wait[i]) in last])
    d = d[(d >= 0) & (d < 50)]
    hop = float(np.median(d)) if d.size else 2.0
    return tile_us, step_us, hop


def measure(out_path, batch=16, prompt_len=496, cap=512, runs=10):
    import torch

    import persistent_megakernel_latency_amd as wpk
    import synth

    cfg = synth.LLAMA_1B
    dev = torch.device("cuda", 0)
    w = synth.make_weights(cfg)
    desc, tensors = wpk.model_from_weights(cfg, w, dev)
    prompt = torch.from_numpy(synth.prompt_tokens(cfg, batch, prompt_len, seed=4).astype(np.int32)).to(dev)
    shape = (cfg.n_layers, batch, cfg.n_kv_heads, cap, cfg.head_dim)
    kc = torch.zeros(shape, dtype=torch.int16, device=dev)
    vc = torch.zeros(shape, dtype=torch.int16, device=dev)
    seq = torch.zeros(batch, dtype=torch.int32, device=dev)
    logits = torch.empty((batch, cfg.vocab), dtype=torch.float32, device=dev)
    tok = torch.empty(batch, dtype=torch.int32, device=dev)
    kv = wpk.wpk_kv(kc.data_ptr(), vc.data_ptr(), seq.data_ptr())
    stream = torch.cuda.current_stream(dev)
    out = {"workload": f"Llama-3.2-1B-shape prefill, batch {batch}, {prompt_len}-token prompts",
           "batch": batch, "prompt": prompt_len, "cap": cap, "measured_us": {}, "source_hash": wpk.prefill_source_hash()}
    for name in DESIGNS:
        plan = wpk.wpk_build_prefill(desc.desc, batch, cap, prompt_len, design_opts(wpk, name))
        if not plan:
            raise RuntimeError(wpk.wpk_prefill_last_error(None))
        info = wpk.wpk_prefill_get_info(plan)

        def go():
            wpk.check_prefill(wpk.wpk_prefill(plan, prompt.data_ptr(), kv, logits.data_ptr(), tok.data_ptr(),
                                              stream.cuda_stream), plan, name)
        for _ in range(2):
            go()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
        for e0, e1 in ev:
            e0.record(stream)
            go()
            e1.record(stream)
        torch.cuda.synchronize(dev)
        wpk.check_prefill(wpk.wpk_prefill_sync(plan), plan, name)
        out["measured_us"][name] = float(np.mean([a.elapsed_time(b) * 1000.0 for a, b in ev]))
        if name == "megakernel":
            wpk.check_prefill(wpk.wpk_prefill_set_option(plan, wpk.WPK_OPT_LOG, 1), plan)
            go()
            wpk.check_prefill(wpk.wpk_prefill_sync(plan), plan, "logged")
            rc, buf = wpk.wpk_prefill_get_log(plan, info.n_tiles)
            wpk.check_prefill(rc, plan, "log")
            log = np.frombuffer(buf, dtype=np.dtype([("exec_count", "<i4"), ("wait_delta", "<i4"), ("worker", "<i4"),
                                                     ("claim", "<i4"), ("t_start", "<i8"), ("t_end", "<i8")]))
            ty, _, wait, signal, _ = (np.array(a) for a in wpk.wpk_prefill_get_dag(plan, info.n_tiles))
            steps = np.array(wpk.wpk_prefill_get_key_steps(plan, info.n_tiles))
            tile_us, step_us, hop = costs_from_log(log, ty, wait, signal, steps)
            out["tile_us"] = {wpk.PREFILL_TILE_TYPES[k]: v for k, v in tile_us.items()}
            out["attn_step_us"] = step_us
            out["hop_us"] = hop
            out["workers"] = info.workers
        wpk.wpk_prefill_destroy(plan)
        print(f"[prefill planner] {name}: {out['measured_us'][name]:.0f} us", file=sys.stderr, flush=True)
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def predict(prof, designs=DESIGNS):
    """Predicted prefill time (µs) of each design from a profile (host only)."""
    import persistent_megakernel_latency_amd as wpk
    import synth

    cfg = synth.LLAMA_1B
    d = _dummy_desc(wpk, cfg)
    res = {}
    for name in designs:
        opts = design_opts(wpk, name)
        if name == "conventional":
            opts = wpk.wpk_prefill_opts(mode=wpk.WPK_PREFILL_MEGAKERNEL)  # the same DAG, run phase by phase
        plan = wpk.wpk_build_prefill_host(d.desc, prof["batch"], prof["cap"], prof["prompt"], opts)
        if not plan:
            raise RuntimeError(wpk.wpk_prefill_last_error(None))
        sp = wpk.wpk_prefill_sim_params()
        for k, n in enumerate(wpk.PREFILL_TILE_TYPES):
            sp.tile_us[k] = float(prof["tile_us"].get(n, 0.0))
        sp.attn_step_us = float(prof["attn_step_us"])
        sp.hop_us = float(prof["hop_us"])
        sp.launch_gap_us = LAUNCH_GAP_US
        sp.workers = int(prof["workers"])
        sp.split_workers = int(name.split("_")[1]) if name.startswith("split_") else 0
        sp.conventional = 1 if name == "conventional" else 0
        rc, r = wpk.wpk_prefill_simulate(plan, sp)
        wpk.wpk_prefill_destroy(plan)
        if rc != 0:
            raise RuntimeError(f"wpk_prefill_simulate: {rc}")
        res[name] = {"predicted_us": r.step_us, "busy": r.worker_busy_frac}
    return res


def _dummy_desc(wpk, cfg):
    """A descriptor with non-null, never dereferenced pointers: host plans
    only build the DAG."""
    fake = 0x1000
    ptrs = {"embed": fake, "final_norm": fake}
    for key in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down"):
        ptrs[key] = [fake] * cfg.n_layers
    return wpk.ModelDesc(cfg, ptrs)


def evaluate(prof):
    """Predictions against the measured times: per-design error, the share
    of design pairs ordered alike, and whether the best design is found."""
    pred = predict(prof)
    meas = prof["measured_us"]
    rows = []
    for n in DESIGNS:
        p, m = pred[n]["predicted_us"], meas[n]
        rows.append({"design": n, "measured_us": m, "predicted_us": p, "error": p / m - 1.0, "busy": pred[n]["busy"]})
    pairs = list(itertools.combinations(DESIGNS, 2))
    agree = sum((pred[a]["predicted_us"] < pred[b]["predicted_us"]) == (meas[a] < meas[b]) for a, b in pairs)
    best_m = min(DESIGNS, key=lambda n: meas[n])
    best_p = min(DESIGNS, key=lambda n: pred[n]["predicted_us"])
    regret = meas[best_p] / meas[best_m] - 1.0
    return {"rows": rows, "pairwise": agree / len(pairs), "pairs": len(pairs), "best_measured": best_m,
            "best_predicted": best_p, "regret": regret}


def markdown(prof, ev):
    lines = ["# Prefill planner: predicted against measured time to first token", "",
             f"Workload: {prof['workload']}; {prof['workers']} workers.  Profile: one logged megakernel prefill "
             f"(per-type median tile times, attention {prof['tile_us'].get('attn', 0):.1f} us + "
             f"{prof['attn_step_us']:.2f} us per 32-key step, hop {prof['hop_us']:.2f} us); launch gap "
             f"{LAUNCH_GAP_US} us.", "",
             "| design | measured (us) | predicted (us) | error | simulated worker busy |", "|---|---|---|---|---|"]
    for r in ev["rows"]:
        lines.append(f"| {r['design']} | {r['measured_us']:.0f} | {r['predicted_us']:.0f} | {100 * r['error']:+.1f}% "
                     f"| {r['busy']:.2f} |")
    lines += ["", f"Pairs ordered alike: {ev['pairwise']:.2f} of {ev['pairs']}; best measured: {ev['best_measured']}, "
              f"best predicted: {ev['best_predicted']} (regret {100 * ev['regret']:.1f}%).", "",
              "Command: `python -m persistent_megakernel_latency_amd.prefill_planner measure --out "
              "profiles/prefill_planner_profile.json` (GPU), then `python -m "
              "persistent_megakernel_latency_amd.prefill_planner validate profiles/prefill_planner_profile.json "
              "--markdown profiles/prefill_planner_validation.md`.", ""]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    m = sub.add_parser("measure")
    m.add_argument("--out", required=True)
    v = sub.add_parser("validate")
    v.add_argument("profile")
    v.add_argument("--markdown")
    a = ap.parse_args()
    if a.cmd == "measure":
        measure(a.out)
        return
    prof = json.load(open(a.profile))
    ev = evaluate(prof)
    print(json.dumps(ev, indent=1))
    if a.markdown:
        with open(a.markdown, "w") as f:
            f.write(markdown(prof, ev))


if __name__ == "__main__":
    main()
