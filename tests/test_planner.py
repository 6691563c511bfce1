"""The planner's simulation (wpk_simulate) on the CPU: closed-form cases and
the orderings its rules imply.  Predictions against measured designs are in
tests/test_planner_validation.py."""
import numpy as np
import pytest

import persistent_megakernel_latency_amd as wpk
import synth
from tests.helpers import dummy_desc


def _plan(cfg, batch, cap, **opts):
    d = dummy_desc(cfg)
    p = wpk.wpk_build_host(d.desc, batch, cap, wpk.wpk_build_opts(**opts) if opts else None)
    assert p, wpk.wpk_last_error(None)
    return p


def _params(workers, bw=1e9, lat=0.0, hop=0.0, gap=0.0, prefetch=1, conventional=0, stage=0.0, compute=0.0, epi=0.0):
    sp = wpk.wpk_sim_params()
    sp.hbm_GBps, sp.load_latency_us, sp.hop_us, sp.launch_gap_us = bw, lat, hop, gap
    sp.workers, sp.prefetch, sp.conventional = workers, prefetch, conventional
    for t in range(wpk.WPK_SIM_TYPES):
        sp.stage_us[t], sp.compute_us[t], sp.epilogue_us[t] = stage, compute, epi
    return sp


def _sim(p, sp, pos=None):
    rc, r = wpk.wpk_simulate(p, sp, pos)
    assert rc == 0
    return r


def test_one_worker_runs_every_tile_in_turn():
    p = _plan(synth.TINY, 1, 64, queue_shards=1)
    n = wpk.wpk_get_info(p).n_tiles
    r = _sim(p, _params(1, stage=0.5, compute=1.0, epi=0.25))
    assert r.step_us == pytest.approx(n * 1.75, rel=1e-6)
    assert r.worker_busy_frac == pytest.approx(1.0, rel=1e-12)
    wpk.wpk_destroy(p)


def test_streaming_bound_with_free_compute():
    cfg = synth.LLAMA_1B
    p = _plan(cfg, 1, 576)
    pos = np.array([496], np.int32)
    r = _sim(p, _params(512, bw=6000.0), pos)
    kv = 16 * 8 * 497 * 64 * 2 * 2
    assert r.hbm_bytes == pytest.approx(cfg.n_matrix_params() * 2 + kv, rel=1e-9)
    # every byte goes through the one server: no faster than bytes / bandwidth
    assert r.step_us >= r.hbm_bytes / 6000e3 * (1 - 1e-12)
    assert r.achieved_GBps <= 6000.0 * (1 + 1e-12)
    wpk.wpk_destroy(p)


def test_dependency_chain_bound_with_unlimited_workers():
    # the tiny DAG per layer: qkv -> attention -> combine -> o-proj -> gate/up
    # -> down, then LM head -> argmax: 6 * 2 + 2 dependent tiles, each 1 us
    # after a 0.5 us hop (the first tiles wait on nothing)
    p = _plan(synth.TINY, 1, 64)
    n = wpk.wpk_get_info(p).n_tiles
    r = _sim(p, _params(4 * n, compute=1.0, hop=0.5))
    chain = 6 * 2 + 2
    assert r.step_us == pytest.approx(chain * 1.0 + (chain - 1) * 0.5, rel=1e-6)
    wpk.wpk_destroy(p)


@pytest.mark.parametrize("batch", [1, 32])
def test_barrier_edges_and_no_prefetch_are_never_faster(batch):
    cfg = synth.LLAMA_1B
    pos = synth.context_lengths(batch) if batch > 1 else np.array([496], np.int32)
    cap = 1152
    fine = _plan(cfg, batch, cap)
    coarse = _plan(cfg, batch, cap, barrier_edges=1)
    base = dict(bw=6200.0, lat=2.0, hop=1.0, stage=1.5, compute=1.0, epi=0.7)
    t_fine = _sim(fine, _params(512, **base), pos).step_us
    t_coarse = _sim(coarse, _params(512, **base), pos).step_us
    t_nopf = _sim(fine, _params(512, prefetch=0, **base), pos).step_us
    assert t_coarse >= t_fine * (1 - 1e-9) and t_nopf >= t_fine * (1 - 1e-9)
    # more bandwidth never hurts
    faster = dict(base, bw=12400.0)
    assert _sim(fine, _params(512, **faster), pos).step_us <= t_fine * (1 + 1e-9)
    wpk.wpk_destroy(fine)
    wpk.wpk_destroy(coarse)


def test_conventional_design_sums_its_operators():
    # one worker, no bandwidth limit: each operator's kernel runs its tiles in
    # turn, then the launch gap before the next
    p = _plan(synth.TINY, 1, 64, queue_shards=1)
    n = wpk.wpk_get_info(p).n_tiles
    ty, layer, _, _ = wpk.wpk_get_dag(p, n)
    phases = 1 + sum(1 for i in range(1, n) if (ty[i], layer[i]) != (ty[i - 1], layer[i - 1]))
    r = _sim(p, _params(1, gap=3.0, conventional=1, compute=1.0))
    assert r.step_us == pytest.approx(n * 1.0 + phases * 3.0, rel=1e-6)
    wpk.wpk_destroy(p)


def test_split_plan_regions_in_the_simulation():
    """A split plan's second megakernel (its last split_workers workers) only
    claims attention and combine tiles: with the same per-tile costs the
    simulated step is no shorter than the single megakernel's, and a worker
    count that leaves a region's queues without a worker is refused."""
    cfg = synth.MINI
    one = _plan(cfg, 8, 140)
    two = _plan(cfg, 8, 140, split_workers=64)
    sp = _params(512, bw=5000.0, lat=2.0, hop=1.0, stage=0.5, compute=1.0, epi=0.5)
    r1, r2 = _sim(one, sp), _sim(two, sp)
    assert r2.step_us >= r1.step_us - 1e-9
    assert r2.hbm_bytes == pytest.approx(r1.hbm_bytes, rel=1e-12)
    rc, _ = wpk.wpk_simulate(two, _params(64 + 4, stage=0.5, compute=1.0, epi=0.5))
    assert rc == wpk.WPK_E_ARG
    wpk.wpk_destroy(one)
    wpk.wpk_destroy(two)
