"""Per-tile timeline of a logged megakernel step, as a trace a person can read.

A logged step (WPK_OPT_LOG) keeps, for every tile, which worker ran it, its
claim position, when its wait ended and when it published, plus a timing
record with the points in between (claimed, inputs staged, weights in,
arithmetic done, partial sums ready).  The pages ask the runtime to record
enough execution state to find where a step went wrong or where its time
went ("Why real-time inference wants a megakernel", "What a megakernel does
not solve": it increases the compiler and verification burden); this module
turns those records into

  * a Chrome/Perfetto trace (JSON "traceEvents"): one process per XCD, one
    thread per worker, one slice per tile with its wait, staging, arithmetic
    and epilogue as nested slices, and flow arrows from the last producer of a
    tile's counter group to the tile;
  * a per-layer phase table: for each operator of a layer, the first tile
    start and last tile end relative to the layer's first QKV start, with the
    median tile duration and the weights streamed.

It reads only what the C ABI returns (wpk_get_log, wpk_get_dag); times are
s_memrealtime ticks of 100 MHz.

    python -m persistent_megakernel_latency_amd.timeline --batch 1 \
        --trace timeline_b1.json.gz --summary profiles/megakernel_llama1b_b1_timeline.md
"""
from __future__ import annotations

import argparse
import ctypes
import gzip
import json
import os
import sys
from typing import Dict, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if os.path.dirname(HERE) not in sys.path:
    sys.path.insert(0, os.path.dirname(HERE))

TICK_US = 0.01  # s_memrealtime runs at 100 MHz

LOG = np.dtype([("exec_count", "<i4"), ("wait_delta", "<i4"), ("worker", "<i4"), ("claim", "<i4"),
                ("t_start", "<i8"), ("t_end", "<i8")])
TIMING = np.dtype([("t_claim", "<i8"), ("t_inputs", "<i8"), ("t_ready", "<i8"), ("t_done", "<i8"),
                   ("t_partials", "<i8"), ("t_end", "<i8"), ("t_stored", "<i8"), ("t_arrived", "<i8")])

TILE_TYPES = ["qkv", "attn", "combine", "oproj", "gateup", "down", "lm", "argmax", "norm", "norm2", "normf",
              "attnc"]
PREFILL_TILE_TYPES = ["embed", "norm1", "qkv", "attn", "oproj", "norm2", "gateup", "down", "normf", "lm", "argmax"]
# operators in the order a layer runs them (the phase table's rows)
PHASE_ORDER = ["embed", "norm", "norm1", "qkv", "attn", "attnc", "combine", "oproj", "norm2", "gateup", "down",
               "normf", "lm", "argmax"]


def split_log(raw: bytes, n_tiles: int, max_workers: int):
    """The three parts of a full wpk_get_log copy: tile records, worker
    records (exec_count = HW_ID, wait_delta = XCC_ID, t_start/t_end = entry
    and exit times) and timing records, or (tile records, None, None) when the
    copy holds only the tile records."""
    raw = bytes(raw)
    rec = np.frombuffer(raw[: n_tiles * LOG.itemsize], dtype=LOG)
    if len(raw) < (2 * n_tiles + max_workers) * LOG.itemsize + n_tiles * LOG.itemsize:
        return rec, None, None
    off = n_tiles * LOG.itemsize
    workers = np.frombuffer(raw[off: off + max_workers * LOG.itemsize], dtype=LOG)
    off += max_workers * LOG.itemsize
    tim = np.frombuffer(raw[off: off + n_tiles * TIMING.itemsize], dtype=TIMING)
    return rec, workers, tim


def read_log(wpk, plan, n_tiles: int, max_workers: int):
    """Copies the last logged step's records of a device plan."""
    nrec = 3 * n_tiles + max_workers
    buf = (wpk.wpk_log_rec * nrec)()
    wpk.check(wpk.lib().wpk_get_log(plan, ctypes.cast(buf, ctypes.c_void_p), ctypes.sizeof(buf)), plan,
              "wpk_get_log")
    return split_log(bytes(buf), n_tiles, max_workers)


def _t0(rec) -> int:
    ran = rec["exec_count"] > 0
    return int(rec["t_start"][ran].min()) if ran.any() else 0


def chrome_trace(rec, dag: Sequence[Sequence[int]], tim=None, workers=None, type_names=TILE_TYPES,
                 flows: bool = True, max_flows: int = 20000) -> Dict[str, object]:
    """The step as Chrome trace events.  dag = (type, layer, wait, signal) per
    tile (wpk_get_dag).  Tiles that did not run are left out."""
    ty, layer, wait, signal = (np.asarray(a) for a in dag)
    n = len(rec)
    t0 = _t0(rec)
    us = lambda t: round((int(t) - t0) * TICK_US, 3)  # noqa: E731
    xcc = {}
    if workers is not None:
        for w in range(len(workers)):
            if workers["worker"][w] == w and workers["t_start"][w] > 0:
                xcc[w] = int(workers["wait_delta"][w])
    ev: List[Dict[str, object]] = []
    pids = sorted(set(xcc.values())) if xcc else [0]
    for p in pids:
        ev.append({"ph": "M", "name": "process_name", "pid": p, "args": {"name": f"XCD {p}" if xcc else "workers"}})
    last_end = {}
    for i in range(n):
        if rec["exec_count"][i] <= 0:
            continue
        w = int(rec["worker"][i])
        pid = xcc.get(w, 0)
        name = f"{type_names[int(ty[i])]} L{int(layer[i])}" if 0 <= int(ty[i]) < len(type_names) else str(int(ty[i]))
        args = {"tile": i, "claim": int(rec["claim"][i]), "wait_group": int(wait[i]), "signal_group": int(signal[i]),
                "wait_delta": int(rec["wait_delta"][i])}
        start, end = int(rec["t_start"][i]), int(rec["t_end"][i])
        if tim is not None and tim["t_claim"][i] > 0 and tim["t_claim"][i] < start:
            ev.append({"ph": "X", "name": "wait", "cat": "wait", "pid": pid, "tid": w, "ts": us(tim["t_claim"][i]),
                       "dur": round((start - int(tim["t_claim"][i])) * TICK_US, 3), "args": {"tile": i}})
        ev.append({"ph": "X", "name": name, "cat": type_names[int(ty[i])] if 0 <= int(ty[i]) < len(type_names) else "?",
                   "pid": pid, "tid": w, "ts": us(start), "dur": round(max(end - start, 0) * TICK_US, 3),
                   "args": args})
        if tim is not None:
            ti, tp = int(tim["t_inputs"][i]), int(tim["t_partials"][i])
            tr = int(tim["t_ready"][i])
            parts = []
            if start <= ti <= end:
                parts.append(("stage inputs", start, ti))
            if ti and tp and ti <= tp <= end:
                parts.append(("compute", max(ti, tr) if tr and tr <= tp else ti, tp))
            if tp and tp <= end:
                parts.append(("epilogue", tp, end))
            for nm, a, b in parts:
                ev.append({"ph": "X", "name": nm, "cat": "part", "pid": pid, "tid": w, "ts": us(a),
                           "dur": round(max(b - a, 0) * TICK_US, 3), "args": {"tile": i}})
        if signal[i] >= 0:
            g = int(signal[i])
            if g not in last_end or end > last_end[g][0]:
                last_end[g] = (end, i)
    if flows:
        nf = 0
        for i in range(n):
            if rec["exec_count"][i] <= 0 or wait[i] < 0 or int(wait[i]) not in last_end or nf >= max_flows:
                continue
            e, src = last_end[int(wait[i])]
            ws, wd = int(rec["worker"][src]), int(rec["worker"][i])
            ev.append({"ph": "s", "id": nf, "name": "ready", "cat": "edge", "pid": xcc.get(ws, 0), "tid": ws,
                       "ts": us(e)})
            ev.append({"ph": "f", "bp": "e", "id": nf, "name": "ready", "cat": "edge", "pid": xcc.get(wd, 0),
                       "tid": wd, "ts": us(rec["t_start"][i])})
            nf += 1
    return {"traceEvents": ev, "displayTimeUnit": "ns",
            "otherData": {"clock": "s_memrealtime, 100 MHz", "t0_ticks": t0}}


def phase_table(rec, dag: Sequence[Sequence[int]], type_names=TILE_TYPES, layers: Optional[Sequence[int]] = None):
    """Per layer and operator: tiles, first start and last end (µs from the
    layer's first QKV start, or its first tile's start when it has no QKV
    tiles) and the median tile duration."""
    ty, layer = np.asarray(dag[0]), np.asarray(dag[1])
    ran = rec["exec_count"] > 0
    qkv = type_names.index("qkv")
    out = {}
    for l in sorted(set(layer[ran].tolist())) if layers is None else layers:
        m = ran & (layer == l)
        if not m.any():
            continue
        q = m & (ty == qkv)
        base = int(rec["t_start"][q].min()) if q.any() else int(rec["t_start"][m].min())
        rows = {}
        for t in sorted(set(ty[m].tolist())):
            mt = m & (ty == t)
            st = rec["t_start"][mt].astype(np.int64)
            en = rec["t_end"][mt].astype(np.int64)
            rows[type_names[t] if 0 <= t < len(type_names) else str(t)] = {
                "tiles": int(mt.sum()),
                "first_start_us": round((int(st.min()) - base) * TICK_US, 2),
                "last_end_us": round((int(en.max()) - base) * TICK_US, 2),
                "median_tile_us": round(float(np.median(en - st)) * TICK_US, 2),
            }
        out[int(l)] = rows
    return out


def type_breakdown(rec, tim, dag, type_names=TILE_TYPES):
    """Per tile type, medians (µs) of: the wait (claimed by the control wave
    until its inputs were complete), input staging, arithmetic (from the
    later of inputs staged and weights in, to the partial sums), the
    epilogue through the publish, and the whole tile.  For a tile of several
    passes (a matrix-core plan's attention tile walks four KV chunks) the
    timing points are those of its last pass, so its staging column also
    covers the earlier passes."""
    ty = np.asarray(dag[0])
    ran = rec["exec_count"] > 0
    out = {}
    for t in sorted(set(ty[ran].tolist())):
        m = ran & (ty == t)
        st, en = rec["t_start"][m].astype(np.int64), rec["t_end"][m].astype(np.int64)
        cl = tim["t_claim"][m].astype(np.int64)
        ti, tr, tp = (tim[k][m].astype(np.int64) for k in ("t_inputs", "t_ready", "t_partials"))
        wait = np.where((cl > 0) & (cl < st), st - cl, 0)
        stage = np.clip(ti - st, 0, None)
        comp = np.clip(tp - np.maximum(ti, np.where(tr <= tp, tr, ti)), 0, None)
        epi = np.clip(en - tp, 0, None)
        med = lambda a: round(float(np.median(a)) * TICK_US, 2)  # noqa: E731
        out[type_names[t] if 0 <= t < len(type_names) else str(t)] = {
            "tiles": int(m.sum()), "wait_us": med(wait), "stage_us": med(stage), "compute_us": med(comp),
            "epilogue_us": med(epi), "tile_us": med(en - st)}
    return out


def layer_spans(rec, dag) -> Dict[int, float]:
    """Per layer: last tile end minus first tile start (µs)."""
    layer = np.asarray(dag[1])
    ran = rec["exec_count"] > 0
    res = {}
    for l in sorted(set(layer[ran].tolist())):
        m = ran & (layer == l)
        res[int(l)] = round((int(rec["t_end"][m].max()) - int(rec["t_start"][m].min())) * TICK_US, 2)
    return res


def markdown_summary(title: str, command: str, table, spans, step_us: float, layers=(1, 7, 14),
                     weights_mb: Optional[Dict[str, float]] = None, breakdown=None, what: str = "step",
                     note: str = "a logged step also waits for each slot's loads before its arithmetic, so it runs "
                                 "slightly slower than a timed one") -> str:
    lines = [f"# {title}", "", "Command (committed files only):", "", "```", command, "```", "",
             f"Logged {what}: {step_us:.1f} µs from the first tile start to the last tile end ({note}).", ""]
    for l in layers:
        if l not in table:
            continue
        lines += [f"## Layer {l} (µs from its first QKV start; layer span {spans.get(l, 0):.1f} µs)", "",
                  "| operator | tiles | first start | last end | median tile | weights (MB) |",
                  "|---|---|---|---|---|---|"]
        rows = table[l]
        for name in PHASE_ORDER + sorted(set(rows) - set(PHASE_ORDER)):
            if name not in rows:
                continue
            r = rows[name]
            wmb = "" if not weights_mb or name not in weights_mb else f"{weights_mb[name]:.1f}"
            lines.append(f"| {name} | {r['tiles']} | {r['first_start_us']:.1f} | {r['last_end_us']:.1f} | "
                         f"{r['median_tile_us']:.2f} | {wmb} |")
        lines.append("")
    if breakdown:
        lines += ["## Per tile type (medians over the step, µs)", "",
                  "Wait: claimed by the control wave until its inputs were complete. Staging: inputs into LDS. "
                  "Arithmetic: from the later of inputs staged and weights in, to the partial sums. A matrix-core "
                  "plan's attention tile walks four KV chunks; its timing points are those of the last pass, so its "
                  "staging column covers the earlier passes too.", "",
                  "| type | tiles | wait | staging | arithmetic | epilogue + publish | tile |", "|---|---|---|---|---|---|---|"]
        for name in PHASE_ORDER + sorted(set(breakdown) - set(PHASE_ORDER)):
            if name in breakdown:
                r = breakdown[name]
                lines.append(f"| {name} | {r['tiles']} | {r['wait_us']:.2f} | {r['stage_us']:.2f} | "
                             f"{r['compute_us']:.2f} | {r['epilogue_us']:.2f} | {r['tile_us']:.2f} |")
        lines.append("")
    if spans:
        vals = [spans[l] for l in sorted(spans) if 0 < l < max(spans)]
        if vals:
            lines += [f"Median layer span over layers 1–{max(spans) - 1}: {float(np.median(vals)):.1f} µs.", ""]
    return "\n".join(lines)


def run(batch: int, trace_path: Optional[str], summary_path: Optional[str], command: str) -> Dict[str, object]:
    """One logged megakernel step of the Llama-3.2-1B-shaped decoder (batch 1:
    a 496-position context; batch above 4: contexts U{256..1024}) after two
    untimed steps, written out as a trace and a phase table."""
    import torch

    import persistent_megakernel_latency_amd as wpk
    import synth

    cfg = synth.LLAMA_1B
    dev = torch.device("cuda", 0)
    desc, tensors = wpk.model_from_weights(cfg, synth.make_weights(cfg), dev)
    if batch == 1:
        lens0 = np.full(1, 496, np.int32)
        tok0 = synth.prompt_tokens(cfg, 1, 496)[:, -1].astype(np.int32)
    else:
        lens0 = synth.context_lengths(batch)
        tok0 = synth.prompt_tokens(cfg, batch, 1)[:, 0].astype(np.int32)
    cap = int(np.ceil((int(lens0.max()) + 8) / 64.0) * 64)
    kc_np, vc_np = synth.synthetic_kv(cfg, batch, cap, lens0)
    kc = torch.from_numpy(kc_np.view(np.int16)).to(dev)
    vc = torch.from_numpy(vc_np.view(np.int16)).to(dev)
    del kc_np, vc_np
    seq = torch.from_numpy(lens0.copy()).to(dev)
    tokens = torch.from_numpy(tok0.copy()).to(dev)
    logits = torch.empty((batch, cfg.vocab), dtype=torch.float32, device=dev)
    kv = wpk.wpk_kv(kc.data_ptr(), vc.data_ptr(), seq.data_ptr())
    plan = wpk.wpk_build(desc.desc, batch, cap)
    if not plan:
        raise RuntimeError("wpk_build: " + wpk.wpk_last_error(None))
    try:
        info = wpk.wpk_get_info(plan)
        for _ in range(2):
            wpk.check(wpk.wpk_step(plan, tokens.data_ptr(), kv, logits.data_ptr(), 0), plan, "wpk_step")
        wpk.check(wpk.wpk_set_option(plan, wpk.WPK_OPT_LOG, 1), plan, "log on")
        wpk.check(wpk.wpk_step(plan, tokens.data_ptr(), kv, logits.data_ptr(), 0), plan, "wpk_step")
        wpk.check(wpk.wpk_sync(plan), plan, "wpk_sync")
        rec, workers, tim = read_log(wpk, plan, info.n_tiles, info.max_workers)
        dag = wpk.wpk_get_dag(plan, info.n_tiles)
    finally:
        wpk.wpk_destroy(plan)
    if not (rec["exec_count"] == 1).all():
        raise RuntimeError("logged step: a tile did not run exactly once")
    ran = rec["exec_count"] > 0
    step_us = (int(rec["t_end"][ran].max()) - int(rec["t_start"][ran].min())) * TICK_US
    table = phase_table(rec, dag)
    spans = layer_spans(rec, dag)
    H, F, D = cfg.hidden, cfg.ffn, cfg.head_dim
    wmb = {"qkv": (cfg.n_q_heads + 2 * cfg.n_kv_heads) * D * H * 2 / 1e6, "oproj": H * H * 2 / 1e6,
           "gateup": 2 * F * H * 2 / 1e6, "down": H * F * 2 / 1e6}
    if trace_path:
        os.makedirs(os.path.dirname(os.path.abspath(trace_path)), exist_ok=True)
        opener = gzip.open if trace_path.endswith(".gz") else open
        with opener(trace_path, "wt") as f:
            json.dump(chrome_trace(rec, dag, tim, workers), f, separators=(",", ":"))
    if summary_path:
        title = f"Per-tile timeline of one logged decode step: Llama-3.2-1B shape, batch {batch}"
        with open(summary_path, "w") as f:
            f.write(markdown_summary(title, command, table, spans, step_us, weights_mb=wmb,
                                     breakdown=type_breakdown(rec, tim, dag)))
    return {"batch": batch, "step_us": round(step_us, 1), "tiles": int(info.n_tiles), "phases": table,
            "layer_span_us": spans}


def run_prefill(trace_path: Optional[str], summary_path: Optional[str], command: str) -> Dict[str, object]:
    """One logged prompt prefill of the Llama-3.2-1B-shaped decoder (batch
    16, 496-token prompts, one megakernel) after one untimed prefill: the
    tile records (the prefill keeps no timing records) as a trace and a
    phase table."""
    import torch

    import persistent_megakernel_latency_amd as wpk
    import synth

    cfg = synth.LLAMA_1B
    dev = torch.device("cuda", 0)
    desc, tensors = wpk.model_from_weights(cfg, synth.make_weights(cfg), dev)
    batch, P, cap = 16, 496, 512
    prompt = torch.from_numpy(synth.prompt_tokens(cfg, batch, P, seed=4).astype(np.int32)).to(dev)
    shape = (cfg.n_layers, batch, cfg.n_kv_heads, cap, cfg.head_dim)
    kc = torch.zeros(shape, dtype=torch.int16, device=dev)
    vc = torch.zeros(shape, dtype=torch.int16, device=dev)
    seq = torch.zeros(batch, dtype=torch.int32, device=dev)
    logits = torch.empty((batch, cfg.vocab), dtype=torch.float32, device=dev)
    tok = torch.empty(batch, dtype=torch.int32, device=dev)
    kv = wpk.wpk_kv(kc.data_ptr(), vc.data_ptr(), seq.data_ptr())
    plan = wpk.wpk_build_prefill(desc.desc, batch, cap, P, wpk.wpk_prefill_opts(mode=wpk.WPK_PREFILL_MEGAKERNEL))
    if not plan:
        raise RuntimeError("wpk_build_prefill: " + wpk.wpk_prefill_last_error(None))
    try:
        info = wpk.wpk_prefill_get_info(plan)
        go = lambda: wpk.check_prefill(wpk.wpk_prefill(plan, prompt.data_ptr(), kv, logits.data_ptr(),  # noqa: E731
                                                       tok.data_ptr(), 0), plan, "wpk_prefill")
        go()
        wpk.check_prefill(wpk.wpk_prefill_set_option(plan, wpk.WPK_OPT_LOG, 1), plan, "log on")
        go()
        wpk.check_prefill(wpk.wpk_prefill_sync(plan), plan, "wpk_prefill_sync")
        rc, log = wpk.wpk_prefill_get_log(plan, info.n_tiles)
        wpk.check_prefill(rc, plan, "wpk_prefill_get_log")
        dag = wpk.wpk_prefill_get_dag(plan, info.n_tiles)[:4]
    finally:
        wpk.wpk_prefill_destroy(plan)
    rec = np.frombuffer(bytes(log), dtype=LOG)
    if not (rec["exec_count"] == 1).all():
        raise RuntimeError("logged prefill: a tile did not run exactly once")
    ran = rec["exec_count"] > 0
    span = (int(rec["t_end"][ran].max()) - int(rec["t_start"][ran].min())) * TICK_US
    table = phase_table(rec, dag, PREFILL_TILE_TYPES)
    spans = layer_spans(rec, dag)
    if trace_path:
        os.makedirs(os.path.dirname(os.path.abspath(trace_path)), exist_ok=True)
        opener = gzip.open if trace_path.endswith(".gz") else open
        with opener(trace_path, "wt") as f:
            json.dump(chrome_trace(rec, dag, type_names=PREFILL_TILE_TYPES), f, separators=(",", ":"))
    if summary_path:
        title = "Per-tile timeline of one logged prompt prefill: Llama-3.2-1B shape, batch 16, 496-token prompts"
        with open(summary_path, "w") as f:
            f.write(markdown_summary(title, command, table, spans, span, what="prefill",
                                     note="one megakernel; a logged prefill records each tile's start and end"))
    return {"prefill": True, "step_us": round(span, 1), "tiles": int(info.n_tiles), "phases": table,
            "layer_span_us": spans}


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--prefill", action="store_true", help="the batch-16 prompt prefill instead of a decode step")
    ap.add_argument("--trace", default=None, help="Chrome/Perfetto trace JSON to write (gzip if it ends in .gz)")
    ap.add_argument("--summary", default=None, help="markdown phase table to write")
    a = ap.parse_args(argv)
    cmd = "python -m persistent_megakernel_latency_amd.timeline " + " ".join(argv if argv is not None else sys.argv[1:])
    res = run_prefill(a.trace, a.summary, cmd) if a.prefill else run(a.batch, a.trace, a.summary, cmd)
    print(json.dumps({"batch": res.get("batch", 16), "step_us": res["step_us"], "tiles": res["tiles"],
                      "median_layer_span_us": float(np.median([v for k, v in res["layer_span_us"].items()
                                                               if 0 < k < max(res["layer_span_us"])]))}))


if __name__ == "__main__":
    main()
