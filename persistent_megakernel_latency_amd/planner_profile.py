"""Per-operator profiles for the planner, and the measured step times it is
checked against (needs a GPU).

For each batch size of the Llama-3.2-1B-shaped decoder it runs one logged
megakernel step of the default design and turns the per-tile timing records
into per-tile-type costs (input staging, compute once the weights are in,
epilogue through the publish: medians over the step's tiles of that type) and
the hop latency (median time from the last producer's publish to a waiting
consumer's start).  It then times the candidate designs on the same inputs:
the megakernel with tile-to-tile edges (default), with barrier edges, without
weight prefetch, with 256 workers, the per-operator hipGraph baseline, and two
co-resident megakernels (attention and combine tiles in one of 128 or 256
workers, every other tile in the other).

    python -m persistent_megakernel_latency_amd.planner_profile --out profiles/planner_profiles.json
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

from persistent_megakernel_latency_amd.timeline import LOG, TIMING  # noqa: E402  (the log's record layouts)


GEMM_TYPES = (0, 3, 4, 5, 6)  # qkv, o-proj, gate/up, down, LM head
SPLITS = (128, 256)  # workers of the attention megakernel in the two-megakernel designs


def tile_costs(wpk, plan, info, wide, hidden, ffn):
    """Per-type (stage, compute, epilogue, row-block reduction) in µs -- the
    medians over the step's tiles of that type; the reduction is what the
    last K slice of a matrix-core row block adds -- and the hop latency, from
    the plan's last logged step."""
    n = info.n_tiles
    nrec = 3 * n + info.max_workers
    buf = (wpk.wpk_log_rec * nrec)()
    wpk.check(wpk.lib().wpk_get_log(plan, ctypes.cast(buf, ctypes.c_void_p), ctypes.sizeof(buf)), plan, "log")
    raw = np.frombuffer(buf, dtype=np.uint8)
    rec = np.frombuffer(raw[: n * 32].tobytes(), dtype=LOG)
    tim = np.frombuffer(raw[(n + info.max_workers) * 32:].tobytes(), dtype=TIMING)[:n]
    ty, _, wait, signal = (np.array(a) for a in wpk.wpk_get_dag(plan, n))
    tick = 0.01  # s_memrealtime: 100 MHz
    costs = {}
    layer = np.array(wpk.wpk_get_dag(plan, n)[1])
    for t in sorted(set(ty.tolist())):
        m = ty == t
        stage = (tim["t_inputs"][m] - rec["t_start"][m]) * tick
        comp = (tim["t_partials"][m] - np.maximum(tim["t_inputs"][m], tim["t_ready"][m])) * tick
        epi = np.maximum((rec["t_end"] - tim["t_partials"]) * tick, 0.0)
        reduce = 0.0
        if wide and t in GEMM_TYPES:
            # the K slices of a row block are consecutive tiles; the one that
            # finishes last has added up the others' partial sums
            nsl = (ffn if t == 5 else hidden) // 512
            red, rest = [], []
            for l in sorted(set(layer[m].tolist())):
                ids = np.nonzero(m & (layer == l))[0]
                for i in range(0, len(ids) - nsl + 1, nsl):
                    run = ids[i:i + nsl]
                    last = run[np.argmax(rec["t_end"][run])]
                    red.append(epi[last])
                    rest.extend(epi[run[run != last]].tolist())
            if red and rest:
                reduce = max(0.0, float(np.median(red)) - float(np.median(rest)))
            epi_t = float(np.median(rest)) if rest else float(np.median(epi[m]))
        else:
            epi_t = float(np.median(epi[m]))
        costs[wpk.TILE_TYPES[t]] = [round(float(np.median(np.maximum(stage, 0.0))), 3),
                                    round(float(np.median(np.maximum(comp, 0.0))), 3), round(epi_t, 3),
                                    round(reduce, 3)]
    last_end = np.full(int(max(wait.max(), signal.max())) + 1, -1, np.int64)
    pm = signal >= 0
    np.maximum.at(last_end, signal[pm], rec["t_end"][pm])
    cons = np.nonzero(wait >= 0)[0]
    waited = cons[tim["t_claim"][cons] < last_end[wait[cons]]]  # claimed before its inputs were complete
    hop = (rec["t_start"][waited] - last_end[wait[waited]]) * tick
    return costs, round(float(np.median(hop)), 3), int(waited.size)


def run(batches, steps, warmup):
    import torch

    import persistent_megakernel_latency_amd as wpk
    import synth

    cfg = synth.LLAMA_1B
    dev = torch.device("cuda", 0)
    desc, tensors = wpk.model_from_weights(cfg, synth.make_weights(cfg), dev)
    out = {"model": cfg.name, "steps": steps, "warmup": warmup, "batches": {}}
    for batch in batches:
        if batch == 1:
            lens0 = np.full(1, 496, np.int32)
            tok0 = synth.prompt_tokens(cfg, 1, 496)[:, -1].astype(np.int32)
        else:
            lens0 = synth.context_lengths(batch)
            tok0 = synth.prompt_tokens(cfg, batch, 1)[:, 0].astype(np.int32)
        cap = int(np.ceil((int(lens0.max()) + warmup + steps + 4) / 64.0) * 64)
        kc_np, vc_np = synth.synthetic_kv(cfg, batch, cap, lens0)
        kc = torch.from_numpy(kc_np.view(np.int16)).to(dev)
        vc = torch.from_numpy(vc_np.view(np.int16)).to(dev)
        del kc_np, vc_np
        seq = torch.from_numpy(lens0.copy()).to(dev)
        tokens = torch.from_numpy(tok0.copy()).to(dev)
        logits = torch.empty((batch, cfg.vocab), dtype=torch.float32, device=dev)
        kv = wpk.wpk_kv(kc.data_ptr(), vc.data_ptr(), seq.data_ptr())
        st = torch.cuda.current_stream(dev)

        def reset():
            seq.copy_(torch.from_numpy(lens0))
            tokens.copy_(torch.from_numpy(tok0))
            torch.cuda.synchronize(dev)

        def timed(plan):
            reset()
            for _ in range(warmup):
                wpk.check(wpk.wpk_step(plan, tokens.data_ptr(), kv, logits.data_ptr(), st.cuda_stream), plan)
            wpk.check(wpk.wpk_sync(plan), plan)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            for a, b in ev:
                a.record(st)
                wpk.check(wpk.wpk_step(plan, tokens.data_ptr(), kv, logits.data_ptr(), st.cuda_stream), plan)
                b.record(st)
            torch.cuda.synchronize(dev)
            wpk.check(wpk.wpk_sync(plan), plan)
            return round(float(np.mean([a.elapsed_time(b) * 1000.0 for a, b in ev])), 2)

        entry = {"positions": (lens0 + warmup).tolist(), "measured_us": {}}
        # profiles: one logged step of the default design, after the warmup
        plan = wpk.wpk_build(desc.desc, batch, cap)
        info = wpk.wpk_get_info(plan)
        reset()
        for _ in range(warmup):
            wpk.check(wpk.wpk_step(plan, tokens.data_ptr(), kv, logits.data_ptr(), st.cuda_stream), plan)
        wpk.check(wpk.wpk_set_option(plan, wpk.WPK_OPT_LOG, 1), plan)
        wpk.check(wpk.wpk_step(plan, tokens.data_ptr(), kv, logits.data_ptr(), st.cuda_stream), plan)
        wpk.check(wpk.wpk_sync(plan), plan)
        entry["costs_us"], entry["hop_us"], entry["hop_samples"] = tile_costs(wpk, plan, info, batch > 4,
                                                                              cfg.hidden, cfg.ffn)
        wpk.check(wpk.wpk_set_option(plan, wpk.WPK_OPT_LOG, 0), plan)
        entry["workers"] = info.workers
        entry["measured_us"]["tile_edges"] = timed(plan)
        wpk.check(wpk.wpk_set_option(plan, wpk.WPK_OPT_PREFETCH, 0), plan)
        entry["measured_us"]["no_prefetch"] = timed(plan)
        wpk.check(wpk.wpk_set_option(plan, wpk.WPK_OPT_PREFETCH, 1), plan)
        wpk.check(wpk.wpk_set_option(plan, wpk.WPK_OPT_WORKERS, 256), plan)
        entry["measured_us"]["workers_256"] = timed(plan)
        wpk.wpk_destroy(plan)
        plan = wpk.wpk_build_ex(desc.desc, batch, cap, wpk.wpk_build_opts(barrier_edges=1))
        entry["measured_us"]["barrier_edges"] = timed(plan)
        wpk.wpk_destroy(plan)
        plan = wpk.wpk_build_graph_baseline(desc.desc, batch, cap)
        entry["measured_us"]["conventional"] = timed(plan)
        wpk.wpk_destroy(plan)
        for w1 in SPLITS:
            plan = wpk.wpk_build_ex(desc.desc, batch, cap, wpk.wpk_build_opts(split_workers=w1))
            entry["measured_us"][f"split_{w1}"] = timed(plan)
            wpk.wpk_destroy(plan)
        out["batches"][str(batch)] = entry
        print(json.dumps({"batch": batch, **entry["measured_us"], "hop_us": entry["hop_us"]}), flush=True)
        del kc, vc
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--batches", default="1,4,8,16,32")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    out = run([int(b) for b in a.batches.split(",")], a.steps, a.warmup)
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
