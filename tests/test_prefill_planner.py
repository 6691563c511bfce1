"""The prefill planner (host only): the design simulator's invariants, and
its predictions against the recorded measurements of the Llama-1B batch-16
496-token prefill (profiles/prefill_planner_profile.json, taken on a GPU by
`prefill_planner measure`)."""
import json
import os

import pytest

import persistent_megakernel_latency_amd as wpk
import synth
from persistent_megakernel_latency_amd import prefill_planner
from tests.helpers import dummy_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILE = os.path.join(ROOT, "profiles", "prefill_planner_profile.json")


def _sim(plan, tile=10.0, step=1.0, hop=0.0, gap=0.0, workers=512, split=0, conv=0):
    sp = wpk.wpk_prefill_sim_params()
    for k in range(11):
        sp.tile_us[k] = tile
    sp.attn_step_us, sp.hop_us, sp.launch_gap_us = step, hop, gap
    sp.workers, sp.split_workers, sp.conventional = workers, split, conv
    return wpk.wpk_prefill_simulate(plan, sp)


def test_prefill_simulator_invariants():
    cfg = synth.MINI
    d = dummy_desc(cfg)
    plan = wpk.wpk_build_prefill_host(d.desc, 2, 300, 257, wpk.wpk_prefill_opts())
    try:
        info = wpk.wpk_prefill_get_info(plan)
        steps = wpk.wpk_prefill_get_key_steps(plan, info.n_tiles)
        ty = wpk.wpk_prefill_get_dag(plan, info.n_tiles)[0]
        # key steps: ceil(min(P, 32 (c + 1)) / 32) per attention tile, 0 elsewhere
        assert all((s > 0) == (t == 3) for s, t in zip(steps, ty))
        assert max(steps) == (257 + 31) // 32
        # one worker per queue: the sum of all tile costs is a lower bound; an
        # unbounded supply of workers makes the critical path the answer
        rc, r1 = _sim(plan, workers=8)
        assert rc == 0
        total = 10.0 * info.n_tiles + sum(steps)
        assert r1.step_us >= total / 8 - 1e-6
        rc, rw = _sim(plan, workers=100000)
        assert rc == 0 and rw.step_us < r1.step_us
        # hops add latency along the critical path only; a larger cost never helps
        rc, rh = _sim(plan, workers=100000, hop=5.0)
        assert rh.step_us > rw.step_us
        rc, rt = _sim(plan, tile=20.0)
        rc, rb = _sim(plan, tile=10.0)
        assert rt.step_us > rb.step_us
        # the conventional design pays one launch gap per phase beyond the first
        rc, c0 = _sim(plan, conv=1, gap=0.0)
        rc, c1 = _sim(plan, conv=1, gap=3.0)
        assert c1.step_us == pytest.approx(c0.step_us + 3.0 * (info.n_phases - 1))
        # refusals: a split pool on a plain plan, too few workers
        assert _sim(plan, split=64)[0] != 0
        assert _sim(plan, workers=4)[0] != 0
    finally:
        wpk.wpk_prefill_destroy(plan)


def test_prefill_planner_against_measurements():
    prof = json.load(open(PROFILE))
    ev = prefill_planner.evaluate(prof)
    rows = {r["design"]: r for r in ev["rows"]}
    # one worker per CU: every design's time follows from the per-tile costs
    for name in prefill_planner.DESIGNS:
        assert abs(rows[name]["error"]) <= 0.2, (name, rows[name])
    assert ev["pairwise"] >= 0.6
    assert ev["regret"] <= 0.05
