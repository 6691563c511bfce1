"""GPU parity: the megakernel (through the C ABI) against the CPU oracle.

Bars: float32 runs max |logit error| <= 1e-4; bf16-weight runs <= 2e-2;
greedy tokens identical (a mismatch is accepted only as a reported near tie,
oracle top-2 margin within 4x the measured error); the canonical per-tile log
(every tile exactly once, counter exactly complete at start) identical to the
serial executor's, and the raw device order a linear extension of the DAG.
"""
import numpy as np
import pytest

import oracle
import persistent_megakernel_latency_amd as wpk
import synth
from tests.gpu_helpers import GpuPlan, announce, tokens_agree
from tests.helpers import check_log

pytestmark = pytest.mark.gpu


def _tiny_prefilled(prompt_len=64, cap=80, gain_std=0.1):
    cfg = synth.TINY
    w = synth.make_weights(cfg, gain_std=gain_std)
    model = oracle.Model(cfg, w)
    prompt = synth.prompt_tokens(cfg, 1, prompt_len)
    kc, vc = model.new_cache(1, cap)
    sl = np.zeros(1, np.int32)
    _, tok = model.prefill(prompt, kc, vc, sl)
    return cfg, w, model, kc, vc, sl, tok


def _teacher_forced(g: GpuPlan, model, kc, vc, sl, tok, steps, tol, name, log=True):
    """Runs `steps` steps feeding the oracle's tokens; returns max logit error."""
    worst = 0.0
    ties = []
    if log:
        wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_LOG, 1), g.plan)
    ty, layer, wait, signal = g.dag()
    for s in range(steps):
        announce(f"{name} step {s}")
        g.set_tokens(tok)
        g.step()
        gk, gv, gsl, gtok, glog = g.state()
        olog, otok = model.step(tok, kc, vc, sl)
        for b in range(len(tok)):
            if sl[b] < 0:
                continue
            err = float(np.max(np.abs(glog[b] - olog[b])))
            worst = max(worst, err)
            assert err <= tol, f"{name} step {s} seq {b}: max |logit err| {err}"
            ok, why = tokens_agree(int(gtok[b]), int(otok[b]), olog[b], err)
            assert ok, f"{name} step {s} seq {b}: {why}"
            if why:
                ties.append(why)
        assert np.array_equal(gsl, sl)
        if log:
            check_log(g.log(), wait, signal)
        tok = otok
    if ties:
        print(f"{name}: near ties {ties}")
    return worst


def test_tiny_fp32_teacher_forced():
    cfg, w, model, kc, vc, sl, tok = _tiny_prefilled()
    g = GpuPlan(cfg, w, 1, kc.shape[3], kc, vc, sl, tok)
    worst = _teacher_forced(g, model, kc, vc, sl, tok, 8, 1e-4, "tiny")
    # the appended keys/values match the oracle's cache at float32 rounding
    gk, gv, _, _, _ = g.state()
    assert np.max(np.abs(gk - kc)) < 1e-5 and np.max(np.abs(gv - vc)) < 1e-5
    print("tiny max logit error", worst)
    g.close()


def test_tiny_free_running_matches_golden_tokens():
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_greedy.json")))
    cfg, w, model, kc, vc, sl, tok = _tiny_prefilled(gold["prompt_len"], gain_std=0.0)
    g = GpuPlan(cfg, w, 1, kc.shape[3], kc, vc, sl, tok)
    got = []
    for s in range(gold["steps"]):
        announce(f"tiny free-running step {s}")
        got.append(int(g.tokens.cpu()[0]))
        g.step()  # tokens chain on the device: no host round trip
    assert got == gold["greedy_tokens"]
    g.close()


def test_mini_bf16_batch_ragged_inactive():
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    model = oracle.Model(cfg, w)
    cap = 200
    lens = np.array([63, -1, 64, 190], np.int32)
    kc, vc = synth.synthetic_kv(cfg, 4, cap, np.maximum(lens, 0))
    tok = np.array([5, 6, 7, 999], np.int32)
    g = GpuPlan(cfg, w, 4, cap, kc, vc, lens, tok)
    k0 = kc.copy()
    worst = _teacher_forced(g, model, kc, vc, lens, tok, 3, 2e-2, "mini-b4")
    gk, gv, gsl, gtok, _ = g.state()
    assert gtok[1] == 6 and gsl[1] == -1
    assert np.array_equal(gk[:, 1], k0[:, 1])
    print("mini max logit error", worst)
    g.close()


@pytest.fixture(scope="module")
def llama():
    cfg = synth.LLAMA_1B
    announce("generating Llama-1B-shaped weights")
    w = synth.make_weights(cfg, gain_std=0.1)
    return cfg, w


LLAMA_CTX, LLAMA_CAP, LLAMA_STEPS = 496, 576, 64


@pytest.fixture(scope="module")
def llama_oracle_run(llama):
    """The oracle's 64 greedy decode steps of the Llama-1B shape at batch 1
    from the 496-position context (positions 496..559): its token before each
    step and its logits at each step."""
    cfg, w = llama
    model = oracle.Model(cfg, w)
    kc, vc = synth.synthetic_kv(cfg, 1, LLAMA_CAP, np.array([LLAMA_CTX]))
    sl = np.array([LLAMA_CTX], np.int32)
    tok = synth.prompt_tokens(cfg, 1, LLAMA_CTX)[:, -1].astype(np.int32).copy()
    k0, v0 = kc.copy(), vc.copy()
    toks, logs = [tok.copy()], []
    for s in range(LLAMA_STEPS):
        announce(f"llama-1b oracle step {s}")
        olog, tok = model.step(tok, kc, vc, sl)
        logs.append(olog[0].copy())
        toks.append(tok.copy())
    return k0, v0, toks, logs


@pytest.mark.timeout(900)
def test_llama_1b_batch1_teacher_forced_all_64_steps(llama, llama_oracle_run):
    """Config 2's 64 decode steps, each fed the oracle's token: logits within
    2e-2, the greedy token, the appended sequence length and the per-tile log
    (every tile once, its counter exactly complete, the device order a linear
    extension of the DAG) at every step."""
    cfg, w = llama
    k0, v0, toks, logs = llama_oracle_run
    announce("llama-1b build")
    g = GpuPlan(cfg, w, 1, LLAMA_CAP, k0, v0, np.array([LLAMA_CTX], np.int32), toks[0])
    wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_LOG, 1), g.plan)
    ty, layer, wait, signal = g.dag()
    worst, ties = 0.0, []
    for s in range(LLAMA_STEPS):
        announce(f"llama-1b teacher-forced step {s}")
        g.set_tokens(toks[s])
        g.step()
        _, _, gsl, gtok, glog = g.state()
        err = float(np.max(np.abs(glog[0] - logs[s])))
        worst = max(worst, err)
        assert err <= 2e-2, f"step {s}: max |logit err| {err}"
        ok, why = tokens_agree(int(gtok[0]), int(toks[s + 1][0]), logs[s], err)
        assert ok, f"step {s}: {why}"
        if why:
            ties.append((s, why))
        assert gsl[0] == LLAMA_CTX + s + 1
        check_log(g.log(), wait, signal)
    print(f"llama-1b 64 teacher-forced steps: max logit error {worst:.3g}, near ties {ties}")
    g.close()


@pytest.mark.timeout(900)
def test_llama_1b_batch1_free_running_64_greedy_tokens(llama, llama_oracle_run):
    """The same 64 steps free-running: the device chains each greedy token
    into the next step with no host round trip, and the sequence must equal
    the oracle's token for token.  Should the two ever part, the step where
    they do must be a near tie (oracle top-2 margin within 4x the measured
    logit error at that step), which is reported; later tokens are then not
    comparable."""
    cfg, w = llama
    k0, v0, toks, logs = llama_oracle_run
    g = GpuPlan(cfg, w, 1, LLAMA_CAP, k0, v0, np.array([LLAMA_CTX], np.int32), toks[0])
    got = []
    for s in range(LLAMA_STEPS):
        announce(f"llama-1b free-running step {s}")
        g.step()
        _, _, _, gtok, glog = g.state()
        got.append(int(gtok[0]))
        if got[-1] != int(toks[s + 1][0]):
            err = float(np.max(np.abs(glog[0] - logs[s])))
            ok, why = tokens_agree(got[-1], int(toks[s + 1][0]), logs[s], err)
            assert ok, f"free-running step {s}: {why}"
            print(f"free-running sequences part at step {s} on a near tie: {why}")
            break
    else:
        assert got == [int(t[0]) for t in toks[1:]]
    g.close()


def _tie_case(batch: int, cap: int = 160):
    """A model in which each sequence's greedy token has an exact twin at a
    lower vocabulary index: the argmax row of the tied embedding is copied onto
    a lower row that no sequence reads as input, so the two logits are the same
    value (bitwise, in the oracle and on the device) and the lower index must
    win."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    rng = np.random.default_rng(7)
    lens = rng.integers(20, cap - 10, size=batch).astype(np.int32)
    kc, vc = synth.synthetic_kv(cfg, batch, cap, lens)
    tok = rng.integers(500, cfg.vocab, size=batch).astype(np.int32)
    model = oracle.Model(cfg, w)
    olog, otok = model.step(tok, kc.copy(), vc.copy(), lens.copy())
    emb = w["embed"].copy()
    used = set(int(t) for t in tok)
    lows = []
    for b in range(batch):
        hi = int(otok[b])
        lo = next(r for r in range(hi - 1, -1, -1) if r not in used and r not in lows and r not in otok)
        emb[lo] = emb[hi]
        lows.append(lo)
    w = dict(w, embed=emb)
    model = oracle.Model(cfg, w)
    olog, otok2 = model.step(tok, kc.copy(), vc.copy(), lens.copy())
    for b in range(batch):
        assert olog[b][lows[b]] == olog[b][int(otok[b])]  # an exact tie in the oracle
        assert otok2[b] == lows[b]                        # its argmax takes the lower index
    return cfg, w, kc, vc, lens, tok, otok, np.array(lows, np.int32), olog


@pytest.mark.parametrize("batch", [2, 8])
def test_device_argmax_exact_tie_takes_the_lower_index(batch):
    """Batch 2 runs the narrow GEMV plan, batch 8 the matrix-core plan."""
    cfg, w, kc, vc, lens, tok, his, lows, olog = _tie_case(batch)
    announce(f"argmax tie batch {batch}")
    g = GpuPlan(cfg, w, batch, kc.shape[3], kc, vc, lens, tok)
    g.step()
    _, _, _, gtok, glog = g.state()
    for b in range(batch):
        # the premise: two identical weight rows give bitwise identical logits
        assert glog[b][lows[b]].tobytes() == glog[b][his[b]].tobytes(), f"seq {b}"
        assert np.max(np.abs(glog[b] - olog[b])) <= 2e-2
        assert int(gtok[b]) == int(lows[b]), f"seq {b}: token {gtok[b]}, tie between {lows[b]} and {his[b]}"
    g.close()


@pytest.mark.parametrize("variant", ["tile16k", "wpc1_q4", "workers200", "cooperative"])
def test_build_and_launch_options_on_the_device(variant):
    """Non-default tile size, worker density, queue count, worker count and
    the cooperative launch, each against the oracle (logits, tokens, log); the
    worker-count and launch variants, which change no arithmetic, are also
    bitwise equal to the default plan."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    model = oracle.Model(cfg, w)
    cap = 200
    lens = np.array([63, 150, 5], np.int32)
    kc, vc = synth.synthetic_kv(cfg, 3, cap, lens)
    tok = np.array([11, 500, 999], np.int32)
    opts = {"tile16k": wpk.wpk_build_opts(tile_bytes=16384),
            "wpc1_q4": wpk.wpk_build_opts(workers_per_cu=1, queue_shards=4)}.get(variant)
    announce(f"options {variant}")
    g = GpuPlan(cfg, w, 3, cap, kc, vc, lens, tok, opts=opts)
    if variant == "workers200":
        wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_WORKERS, 200), g.plan)
    if variant == "cooperative":
        wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_LAUNCH, 1), g.plan)
    ref = GpuPlan(cfg, w, 3, cap, kc, vc, lens, tok, desc=g.desc) if variant in ("workers200", "cooperative") else None
    okc, ovc, osl = kc.copy(), vc.copy(), lens.copy()
    _teacher_forced(g, model, okc, ovc, osl, tok, 3, 2e-2, f"options {variant}")
    if ref is not None:
        g2 = GpuPlan(cfg, w, 3, cap, kc, vc, lens, tok, desc=g.desc)
        if variant == "workers200":
            wpk.check(wpk.wpk_set_option(g2.plan, wpk.WPK_OPT_WORKERS, 200), g2.plan)
        else:
            wpk.check(wpk.wpk_set_option(g2.plan, wpk.WPK_OPT_LAUNCH, 1), g2.plan)
        for _ in range(3):
            g2.step()
            ref.step()
        for x, y in zip(g2.state(), ref.state()):
            assert np.array_equal(x, y)
        g2.close()
        ref.close()
    g.close()


def test_graph_baseline_equals_megakernel_bitwise():
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    cap = 130
    lens = np.array([100, 7], np.int32)
    kc, vc = synth.synthetic_kv(cfg, 2, cap, lens)
    tok = np.array([1, 2], np.int32)
    announce("mini megakernel vs hipGraph baseline")
    a = GpuPlan(cfg, w, 2, cap, kc, vc, lens, tok)
    b = GpuPlan(cfg, w, 2, cap, kc, vc, lens, tok, baseline=True, desc=a.desc)
    for s in range(3):
        a.step()
        b.step()
        sa, sb = a.state(), b.state()
        for x, y in zip(sa, sb):
            assert np.array_equal(x, y), f"step {s}"
    a.close()
    b.close()


@pytest.mark.parametrize("plan", ["tiny", "mini-wide"])
def test_determinism_perturbation_and_prefetch_off(plan):
    """Run-to-run bitwise determinism of the narrow (tiny, batch 1) and the
    matrix-core (MINI, batch 8) plans: repeated runs, runs with random delays
    before each tile (other claim and completion orders) and runs without the
    weight prefetch give the same bits."""
    if plan == "tiny":
        cfg, w, model, kc, vc, sl, tok = _tiny_prefilled(prompt_len=30, cap=64)
        batch, cap = 1, 64
    else:
        cfg = synth.MINI
        w = synth.make_weights(cfg, gain_std=0.1)
        batch, cap = 8, 140
        sl = np.array([63, 64, 65, 1, 100, 128, 129, 7], np.int32)
        kc, vc = synth.synthetic_kv(cfg, batch, cap, sl)
        tok = np.arange(1, batch + 1, dtype=np.int32) * 97
    outs = []
    for variant in ("base", "again", "perturb", "noprefetch"):
        announce(f"{plan} determinism {variant}")
        g = GpuPlan(cfg, w, batch, cap, kc, vc, sl, tok)
        if variant == "perturb":
            wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_PERTURB_SEED, 1234), g.plan)
        if variant == "noprefetch":
            wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_PREFETCH, 0), g.plan)
        for _ in range(3):
            g.step()
        outs.append(g.state())
        g.close()
    for o in outs[1:]:
        for x, y in zip(outs[0], o):
            assert np.array_equal(x, y)


def test_watchdog_reports_a_missing_publish_and_recovers():
    cfg, w, model, kc, vc, sl, tok = _tiny_prefilled(prompt_len=20, cap=64)
    g = GpuPlan(cfg, w, 1, 64, kc, vc, sl, tok)
    ty, layer, wait, signal = g.dag()
    victim = next(i for i in range(len(ty)) if ty[i] == 4 and layer[i] == 0)  # a gate/up tile
    wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_WATCHDOG_US, 20000), g.plan)
    wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_DEBUG_DROP_TILE, victim), g.plan)
    announce("tiny watchdog (dropped publish)")
    rc = g.step(check=False)
    assert rc == wpk.WPK_E_TIMEOUT
    msg = wpk.wpk_last_error(g.plan)
    assert "tile" in msg
    # the tile that timed out is blocked (directly or downstream) by the victim,
    # and the root cause reported is the victim's counter group, one publish short
    named = int(msg.split("tile ")[1].split()[0])
    assert wait[named] >= signal[victim]
    group = int(msg.split("first incomplete group ")[1].split(":")[0])
    assert group == signal[victim]
    producers = sum(1 for s in signal if s == group)
    assert f"{producers - 1} of {producers} publishes" in msg
    assert wpk.wpk_step(g.plan, g.tokens.data_ptr(), g.kv, g.logits.data_ptr(), 0) == wpk.WPK_E_STATE
    # reset, restore the inputs, run clean
    wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_DEBUG_DROP_TILE, -1), g.plan)
    wpk.check(wpk.wpk_set_option(g.plan, wpk.WPK_OPT_RESET, 1), g.plan)
    g2 = GpuPlan(cfg, w, 1, 64, kc, vc, sl, tok)
    g.kc.copy_(g2.kc)
    g.vc.copy_(g2.vc)
    g.seq_len.copy_(g2.seq_len)
    g.set_tokens(tok)
    announce("tiny after reset")
    g.step()
    g2.step()
    for x, y in zip(g.state(), g2.state()):
        assert np.array_equal(x, y)
    g.close()
    g2.close()
