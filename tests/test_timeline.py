"""CPU tests of the per-tile timeline exporter: a trace of the threaded
protocol emulator's step (real claim order and times), and synthetic device
records with timing points."""
import json

import numpy as np

import oracle
import persistent_megakernel_latency_amd as wpk
import synth
from persistent_megakernel_latency_amd import timeline as tl
from tests.helpers import HostState, host_desc


def _emulated_step(threads=8, seed=1, serial=False):
    cfg = synth.TINY
    w = synth.make_weights(cfg, gain_std=0.1)
    model = oracle.Model(cfg, w)
    kc, vc = model.new_cache(1, 40)
    sl = np.zeros(1, np.int32)
    _, tok = model.prefill(synth.prompt_tokens(cfg, 1, 16), kc, vc, sl)
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, 1, kc.shape[3])
    assert plan, wpk.wpk_last_error(None)
    n = wpk.wpk_get_info(plan).n_tiles
    st = HostState(kc, vc, sl, tok, cfg.vocab)
    rc = st.serial(plan, seed) if serial else st.emulate(plan, threads, seed)
    assert rc == 0, wpk.wpk_last_error(plan)
    rc, log = wpk.wpk_get_log(plan, n)
    assert rc == 0
    dag = wpk.wpk_get_dag(plan, n)
    wpk.wpk_destroy(plan)
    rec, workers, tim = tl.split_log(bytes(log), n, 0)
    return rec, dag, cfg


def test_trace_of_an_emulated_step_has_every_tile_and_ordered_edges():
    rec, dag, cfg = _emulated_step()
    ty, layer, wait, signal = (np.asarray(a) for a in dag)
    n = len(rec)
    tr = tl.chrome_trace(rec, dag)
    json.dumps(tr)  # serialisable
    tiles = [e for e in tr["traceEvents"] if e["ph"] == "X" and e["cat"] not in ("part", "wait")]
    assert sorted(e["args"]["tile"] for e in tiles) == list(range(n))
    for e in tiles:
        i = e["args"]["tile"]
        assert e["name"] == f"{tl.TILE_TYPES[ty[i]]} L{layer[i]}"
        assert e["tid"] == int(rec["worker"][i]) and e["dur"] >= 0
        assert e["args"]["wait_group"] == wait[i] and e["args"]["signal_group"] == signal[i]
    # one flow arrow per waiting tile, from its group's last producer, never
    # pointing back in time (the emulator's order is a linear extension)
    starts = {e["id"]: e for e in tr["traceEvents"] if e["ph"] == "s"}
    ends = {e["id"]: e for e in tr["traceEvents"] if e["ph"] == "f"}
    assert set(starts) == set(ends) and len(starts) == int(np.sum(wait >= 0))
    for k in starts:
        assert starts[k]["ts"] <= ends[k]["ts"]


def test_phase_table_orders_a_layers_operators():
    # the serial executor: one tile at a time, in a seeded topological order
    rec, dag, cfg = _emulated_step(seed=3, serial=True)
    table = tl.phase_table(rec, dag)
    assert sorted(table) == list(range(cfg.n_layers))
    for l, rows in table.items():
        assert rows["qkv"]["first_start_us"] == 0.0
        for r in rows.values():
            assert r["first_start_us"] <= r["last_end_us"] and r["tiles"] > 0
        # operators whose every tile needs all of the previous one's tiles
        assert rows["combine"]["last_end_us"] <= rows["oproj"]["first_start_us"]
        assert rows["oproj"]["last_end_us"] <= rows["gateup"]["first_start_us"]
        assert rows["gateup"]["last_end_us"] <= rows["down"]["first_start_us"]
    ty = np.asarray(dag[0])
    assert sum(r["tiles"] for rows in table.values() for r in rows.values()) == len(ty)
    spans = tl.layer_spans(rec, dag)
    md = tl.markdown_summary("t", "cmd", table, spans, 1.0, layers=(0, 1))
    assert "| qkv |" in md and "Layer 1" in md


def test_split_log_and_nested_parts_from_device_records():
    n, mw = 3, 4
    rec = np.zeros(n, tl.LOG)
    rec["exec_count"] = 1
    rec["worker"] = [0, 1, 1]
    rec["claim"] = [0, 0, 1]
    rec["t_start"] = [1000, 1300, 1600]
    rec["t_end"] = [1200, 1500, 1900]
    workers = np.zeros(mw, tl.LOG)
    workers["worker"] = np.arange(mw)
    workers["t_start"] = [900, 900, 0, 0]  # two workers ran
    workers["wait_delta"] = [3, 5, 0, 0]   # their XCDs
    tim = np.zeros(n, tl.TIMING)
    tim["t_claim"] = [950, 1300, 1510]
    tim["t_inputs"] = [1050, 1350, 1650]
    tim["t_ready"] = [1040, 1360, 1640]
    tim["t_partials"] = [1150, 1450, 1850]
    raw = rec.tobytes() + workers.tobytes() + tim.tobytes()
    r2, w2, t2 = tl.split_log(raw, n, mw)
    assert np.array_equal(r2, rec) and np.array_equal(w2, workers) and np.array_equal(t2, tim)
    # only the tile records: no timing
    r3, w3, t3 = tl.split_log(rec.tobytes(), n, mw)
    assert w3 is None and t3 is None and np.array_equal(r3, rec)
    dag = ([0, 1, 3], [0, 0, 0], [-1, 0, 1], [0, 1, -1])
    tr = tl.chrome_trace(r2, dag, t2, w2)
    ev = tr["traceEvents"]
    names = {e["args"]["name"] for e in ev if e["ph"] == "M"}
    assert names == {"XCD 3", "XCD 5"}
    tile1 = next(e for e in ev if e["ph"] == "X" and e.get("args", {}).get("tile") == 1 and e.get("cat") == "attn")
    assert tile1["pid"] == 5 and tile1["ts"] == 3.0 and tile1["dur"] == 2.0  # 100 MHz ticks from t0 = 1000
    parts = {e["name"]: e for e in ev if e.get("cat") == "part" and e["args"]["tile"] == 1}
    assert parts["stage inputs"]["ts"] == 3.0 and parts["stage inputs"]["dur"] == 0.5
    assert parts["compute"]["ts"] == 3.6 and parts["compute"]["dur"] == 0.9  # from the weights' arrival
    assert parts["epilogue"]["ts"] == 4.5 and parts["epilogue"]["dur"] == 0.5
    waits = [e for e in ev if e.get("cat") == "wait"]
    assert {e["args"]["tile"] for e in waits} == {0, 2}  # tile 1 was claimed at its start
    assert next(e for e in waits if e["args"]["tile"] == 2)["dur"] == 0.9
    bd = tl.type_breakdown(r2, t2, dag)
    assert bd["attn"] == {"tiles": 1, "wait_us": 0.0, "stage_us": 0.5, "compute_us": 0.9, "epilogue_us": 0.5,
                          "tile_us": 2.0}
    assert bd["oproj"]["wait_us"] == 0.9 and bd["qkv"]["compute_us"] == 1.0  # weights in before the inputs
    md = tl.markdown_summary("t", "cmd", tl.phase_table(r2, dag), {}, 1.0, layers=(0,), breakdown=bd)
    assert "| attn | 1 | 0.00 | 0.50 | 0.90 | 0.50 | 2.00 |" in md
    # flows: tile 0 -> tile 1 and tile 1 -> tile 2
    s = sorted((e["ts"], e["tid"]) for e in ev if e["ph"] == "s")
    f = sorted((e["ts"], e["tid"]) for e in ev if e["ph"] == "f")
    assert s == [(2.0, 0), (5.0, 1)] and f == [(3.0, 1), (6.0, 1)]


def test_prefill_phase_table_on_a_prefill_dag():
    """The prefill's tile types and layers, with synthetic times in tile-id
    order (a topological order of the prefill DAG)."""
    from tests.helpers import dummy_desc
    cfg = synth.MINI
    d = dummy_desc(cfg)
    plan = wpk.wpk_build_prefill_host(d.desc, 2, 64, 48, wpk.wpk_prefill_opts(mode=wpk.WPK_PREFILL_MEGAKERNEL))
    assert plan, wpk.wpk_prefill_last_error(None)
    n = wpk.wpk_prefill_get_info(plan).n_tiles
    dag = wpk.wpk_prefill_get_dag(plan, n)[:4]
    wpk.wpk_prefill_destroy(plan)
    rec = np.zeros(n, tl.LOG)
    rec["exec_count"] = 1
    rec["t_start"] = 100 * np.arange(n)
    rec["t_end"] = 100 * np.arange(n) + 50
    table = tl.phase_table(rec, dag, tl.PREFILL_TILE_TYPES)
    assert sorted(table) == list(range(cfg.n_layers))
    for l, rows in table.items():
        assert rows["qkv"]["first_start_us"] == 0.0
        assert rows["qkv"]["last_end_us"] <= rows["oproj"]["last_end_us"] <= rows["down"]["last_end_us"]
        assert all(r["median_tile_us"] == 0.5 for r in rows.values())
    assert "embed" in table[0] and "lm" in table[cfg.n_layers - 1]
    tr = tl.chrome_trace(rec, dag, type_names=tl.PREFILL_TILE_TYPES, flows=False)
    assert sum(1 for e in tr["traceEvents"] if e["ph"] == "X") == n
