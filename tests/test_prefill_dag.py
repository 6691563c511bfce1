"""The prompt-prefill DAG on the host (no GPU): shape, coverage, claim order,
queues of the split plan, and the shapes the builder refuses.

The DAG is checked here independently of the builder's own validation: the
tile counts per type are recomputed from the model and prompt, every tile's
wait group must be produced by tiles earlier in claim order, and a Kahn-style
replay of the counter groups must run every tile exactly once.
"""
import math

import numpy as np
import pytest

import persistent_megakernel_latency_amd as wpk
import synth
from tests.helpers import dummy_desc

T = {name: i for i, name in enumerate(wpk.PREFILL_TILE_TYPES)}


def _host(cfg, batch, cap, prompt, mode=0, split_workers=0):
    d = dummy_desc(cfg)
    opts = wpk.wpk_prefill_opts(mode=mode, split_workers=split_workers)
    plan = wpk.wpk_build_prefill_host(d.desc, batch, cap, prompt, opts)
    assert plan, wpk.wpk_prefill_last_error(None)
    return plan


def _expected_counts(cfg, batch, prompt):
    nrb = batch * math.ceil(prompt / 128)
    nqb = math.ceil(prompt / 64)
    L = cfg.n_layers
    return {
        "embed": 8 * nrb, "norm1": 8 * (L - 1) * nrb, "qkv": L * nrb * cfg.qkv_rows // 256,
        "attn": L * batch * nqb * cfg.n_kv_heads, "oproj": L * nrb * cfg.hidden // 256, "norm2": 8 * L * nrb,
        "gateup": L * nrb * cfg.ffn // 128, "down": L * nrb * cfg.hidden // 256, "normf": batch,
        "lm": math.ceil(cfg.vocab / 256), "argmax": 1,
    }


def _replay(ty, wait, signal):
    """Counter-group replay in claim order: each tile runs when every producer
    of its group has run; returns the run order (all tiles, each once)."""
    n = len(ty)
    producers = {}
    for u, s in enumerate(signal):
        if s >= 0:
            producers.setdefault(s, 0)
            producers[s] += 1
    done = {g: 0 for g in producers}
    ran = np.zeros(n, bool)
    order = []
    for v in range(n):  # claim order is a topological order
        g = wait[v]
        assert g < 0 or done.get(g, -1) == producers[g], f"tile {v} claimed before its group {g} completed"
        ran[v] = True
        order.append(v)
        if signal[v] >= 0:
            done[signal[v]] += 1
    assert ran.all()
    return order


@pytest.mark.parametrize("cfg,batch,prompt", [(synth.LLAMA_1B, 16, 496), (synth.MINI, 3, 150), (synth.MINI, 1, 1),
                                              (synth.MINI, 5, 128)])
def test_prefill_dag_shape_and_order(cfg, batch, prompt):
    plan = _host(cfg, batch, 1024 if prompt > 200 else 200, prompt)
    try:
        info = wpk.wpk_prefill_get_info(plan)
        ty, layer, wait, signal, queue = wpk.wpk_prefill_get_dag(plan, info.n_tiles)
        want = _expected_counts(cfg, batch, prompt)
        got = {name: int(np.sum(np.asarray(ty) == T[name])) for name in want}
        assert got == want
        assert info.n_tiles == sum(want.values())
        assert info.rows_per_sequence == 128 * math.ceil(prompt / 128)
        _replay(ty, wait, signal)
        # claim queues: each in claim order; row-block tiles of one row block share a queue
        # (small prompts may leave some of the eight queues empty: their workers exit at once)
        q = np.asarray(queue)
        assert q.min() == 0 and q.max() < info.n_queues == 8
        if batch * math.ceil(prompt / 128) >= 8:
            assert len(set(q.tolist())) == 8
        # phases of the per-operator baseline: one per (layer, type) run
        runs = 1 + int(np.sum((np.diff(ty) != 0) | (np.diff(layer) != 0)))
        assert info.n_phases == runs == 7 * cfg.n_layers + 3
        # the matrix-product FLOPs
        rows = batch * prompt
        per_row = 2 * (cfg.qkv_rows * cfg.hidden + cfg.hidden * cfg.hidden + 3 * cfg.ffn * cfg.hidden)
        attn = 4 * prompt * (prompt + 1) / 2 * 64 * cfg.n_q_heads * batch
        flops = cfg.n_layers * (rows * per_row + attn) + 2 * batch * cfg.vocab * cfg.hidden
        assert info.flops == pytest.approx(flops, rel=1e-12)
    finally:
        wpk.wpk_prefill_destroy(plan)


def test_prefill_dag_edges_follow_row_blocks():
    """Each consumer waits on exactly the producers of what it reads: QKV on
    its row block's norm, attention on every QKV tile of its sequence, the
    o-projection on the attention tiles of its row block, and so on."""
    cfg, batch, prompt = synth.MINI, 2, 200  # two row blocks, the second ragged
    plan = _host(cfg, batch, 256, prompt)
    try:
        info = wpk.wpk_prefill_get_info(plan)
        ty, layer, wait, signal, queue = wpk.wpk_prefill_get_dag(plan, info.n_tiles)
        ty, wait, signal, layer = map(np.asarray, (ty, wait, signal, layer))
        prod = {}
        for u in range(info.n_tiles):
            if signal[u] >= 0:
                prod.setdefault(int(signal[u]), []).append(u)
        nrb_s = 2
        per = {"qkv": 8, "attn": nrb_s * cfg.qkv_rows // 256, "norm2": cfg.hidden // 256,
               "gateup": 8, "down": cfg.ffn // 128, "norm1": cfg.hidden // 256, "lm": batch,
               "argmax": math.ceil(cfg.vocab / 256), "normf": cfg.hidden // 256}
        src = {"qkv": ("embed", "norm1"), "attn": ("qkv",), "oproj": ("attn",), "norm2": ("oproj",),
               "gateup": ("norm2",), "down": ("gateup",), "norm1": ("down",), "normf": ("down",), "lm": ("normf",),
               "argmax": ("lm",)}
        for v in range(info.n_tiles):
            name = wpk.PREFILL_TILE_TYPES[ty[v]]
            if wait[v] < 0:
                assert name == "embed"
                continue
            ps = prod[int(wait[v])]
            assert all(wpk.PREFILL_TILE_TYPES[ty[p]] in src[name] for p in ps), (v, name)
            assert max(ps) < v
            if name in per:
                assert len(ps) == per[name], (v, name, len(ps))
            else:  # oproj: the attention tiles of the row block (2 query blocks x kv heads, 1 if ragged)
                assert len(ps) in tuple(k * cfg.n_kv_heads for k in (1, 2))
            lay = {"norm1": -1}.get(name, 0)
            if name not in ("lm", "argmax", "normf"):
                assert all(layer[p] == layer[v] + lay for p in ps)
    finally:
        wpk.wpk_prefill_destroy(plan)


def test_prefill_split_plan_queues():
    """Split plans: the attention tiles, and only those, sit in the second
    region's queues."""
    cfg = synth.LLAMA_1B
    plan = _host(cfg, 16, 512, 496, mode=wpk.WPK_PREFILL_SPLIT)
    try:
        info = wpk.wpk_prefill_get_info(plan)
        ty, layer, wait, signal, queue = map(np.asarray, wpk.wpk_prefill_get_dag(plan, info.n_tiles))
        assert info.n_queues == 16
        attn = ty == T["attn"]
        assert np.all(queue[attn] >= 8) and np.all(queue[~attn] < 8)
        _replay(list(ty), list(wait), list(signal))
    finally:
        wpk.wpk_prefill_destroy(plan)


@pytest.mark.parametrize("what", ["f32", "prompt0", "prompt_gt_cap", "batch33", "split_workers_nonsplit", "mode"])
def test_prefill_refusals(what):
    cfg, batch, cap, prompt, opts = synth.MINI, 2, 128, 64, wpk.wpk_prefill_opts()
    if what == "f32":
        cfg = synth.TINY
    elif what == "prompt0":
        prompt = 0
    elif what == "prompt_gt_cap":
        prompt = cap + 1
    elif what == "batch33":
        batch = 33
    elif what == "split_workers_nonsplit":
        opts = wpk.wpk_prefill_opts(mode=0, split_workers=16)
    else:
        opts = wpk.wpk_prefill_opts(mode=3)
    d = dummy_desc(cfg)
    plan = wpk.wpk_build_prefill_host(d.desc, batch, cap, prompt, opts)
    assert not plan
    assert wpk.wpk_prefill_last_error(None)
