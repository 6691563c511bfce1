"""CPU tests of the tile-graph builder, the serial DAG executor, the threaded
protocol emulator and the C-ABI surface (no GPU)."""
import ctypes

import numpy as np
import pytest

import oracle
import persistent_megakernel_latency_amd as wpk
import synth
from tests.helpers import HostState, check_log, dummy_desc, header_symbols, host_desc


def test_library_exports_every_declared_symbol():
    declared = header_symbols()
    assert "wpk_build" in declared and "wpk_step" in declared
    lib = wpk.lib()
    missing = [s for s in declared if not hasattr(lib, s)]
    assert missing == []
    assert sorted(wpk.symbols()) == declared


def test_build_errors_are_reported():
    d = dummy_desc(synth.TINY)
    assert not wpk.wpk_build_host(d.desc, 0, 64)
    assert "batch" in wpk.wpk_last_error(None)
    d.desc.head_dim = 32
    assert not wpk.wpk_build_host(d.desc, 1, 64)
    assert "head_dim" in wpk.wpk_last_error(None)


def _info_and_dag(cfg, batch, cap, **opts):
    d = dummy_desc(cfg)
    o = wpk.wpk_build_opts(**opts) if opts else None
    p = wpk.wpk_build_host(d.desc, batch, cap, o)
    assert p, wpk.wpk_last_error(None)
    info = wpk.wpk_get_info(p)
    dag = wpk.wpk_get_dag(p, info.n_tiles)
    wpk.wpk_destroy(p)
    return info, dag


def test_llama_1b_dag_shape():
    cfg = synth.LLAMA_1B
    info, (ty, layer, wait, signal) = _info_and_dag(cfg, 1, 576)
    ty = np.array(ty)
    # per layer: QKV 3072/16 = 192, attention 8 kv heads x 9 chunks, 8 combines,
    # o-proj 2048/16, gate/up 8192/8, down 2048/4; then 128256/16 LM tiles + argmax
    per_layer = {0: 192, 1: 72, 2: 8, 3: 128, 4: 1024, 5: 512}
    for t, n in per_layer.items():
        assert np.sum(ty == t) == 16 * n
    assert np.sum(ty == 6) == 8016 and np.sum(ty == 7) == 1
    assert info.n_tiles == 16 * sum(per_layer.values()) + 8016 + 1
    assert info.rows_per_tile_h == 16 and info.rows_per_tile_f == 4
    assert info.weight_bytes == synth.LLAMA_1B.weight_bytes()
    # every consumer's producers precede it (the claim order is topological)
    last_prod = {}
    for u, s in enumerate(signal):
        if s >= 0:
            last_prod[s] = u
    for v, g in enumerate(wait):
        if g >= 0:
            assert last_prod[g] < v


@pytest.mark.parametrize("tile_bytes", [4096, 16384, 65536])
def test_dag_validates_for_tile_sizes(tile_bytes):
    for cfg in (synth.TINY, synth.MINI):
        info, _ = _info_and_dag(cfg, 2, 100, tile_bytes=tile_bytes)
        assert info.n_tiles > 0


def _tiny_setup(prompt_len=16, cap=40, gain_std=0.1):
    cfg = synth.TINY
    w = synth.make_weights(cfg, gain_std=gain_std)
    model = oracle.Model(cfg, w)
    prompt = synth.prompt_tokens(cfg, 1, prompt_len)
    kc, vc = model.new_cache(1, cap)
    sl = np.zeros(1, np.int32)
    _, tok = model.prefill(prompt, kc, vc, sl)
    return cfg, w, model, kc, vc, sl, tok


def test_serial_executor_matches_oracle_and_is_order_independent():
    cfg, w, model, kc, vc, sl, tok = _tiny_setup()
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, 1, kc.shape[3])
    assert plan, wpk.wpk_last_error(None)
    n = wpk.wpk_get_info(plan).n_tiles
    _, _, wait, signal = wpk.wpk_get_dag(plan, n)
    ref_state = None
    for step in range(3):
        # the oracle's step (teacher-forced input tok)
        ok_, ov_, osl = kc.copy(), vc.copy(), sl.copy()
        olog, otok = model.step(tok, ok_, ov_, osl)
        results = []
        for seed in range(100):
            st = HostState(kc, vc, sl, tok, cfg.vocab)
            assert st.serial(plan, seed, poison=(seed % 2 == 1)) == 0, wpk.wpk_last_error(plan)
            rc, log = wpk.wpk_get_log(plan, n)
            assert rc == 0
            check_log(log, wait, signal)
            results.append(st)
        for st in results[1:]:
            assert np.array_equal(st.logits, results[0].logits)
            assert np.array_equal(st.kc, results[0].kc) and np.array_equal(st.vc, results[0].vc)
        st = results[0]
        assert np.max(np.abs(st.logits[0] - olog[0])) < 1e-4
        assert st.tokens[0] == otok[0] and st.seq_len[0] == osl[0]
        kc, vc, sl, tok = ok_, ov_, osl, otok  # continue from the oracle's state


def test_dropped_edge_is_caught_by_nan_poison():
    cfg, w, model, kc, vc, sl, tok = _tiny_setup()
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, 1, kc.shape[3])
    n = wpk.wpk_get_info(plan).n_tiles
    ty, layer, wait, signal = wpk.wpk_get_dag(plan, n)
    # an output-projection tile of layer 1 no longer waits for the attention combine
    victim = next(i for i in range(n) if ty[i] == 3 and layer[i] == 1)
    assert wpk.wpk_debug_drop_edge(plan, victim) == 0
    poisoned = 0
    for seed in range(8):
        st = HostState(kc, vc, sl, tok, cfg.vocab)
        st.serial(plan, seed, poison=True)
        poisoned += int(np.isnan(st.logits).any())
    assert poisoned > 0
    assert wpk.wpk_debug_drop_edge(plan, -1) == 0
    st = HostState(kc, vc, sl, tok, cfg.vocab)
    assert st.serial(plan, 0, poison=True) == 0 and not np.isnan(st.logits).any()
    wpk.wpk_destroy(plan)


@pytest.mark.parametrize("threads", [8, 33])
def test_emulated_protocol_matches_serial(threads):
    cfg, w, model, kc, vc, sl, tok = _tiny_setup()
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, 1, kc.shape[3])
    n = wpk.wpk_get_info(plan).n_tiles
    _, _, wait, signal = wpk.wpk_get_dag(plan, n)
    ref = HostState(kc, vc, sl, tok, cfg.vocab)
    assert ref.serial(plan, 0) == 0
    for seed in range(3):
        st = HostState(kc, vc, sl, tok, cfg.vocab)
        assert st.emulate(plan, threads, seed) == 0, wpk.wpk_last_error(plan)
        rc, log = wpk.wpk_get_log(plan, n)
        check_log(log, wait, signal)
        assert np.array_equal(st.logits, ref.logits)
        assert st.tokens[0] == ref.tokens[0] and st.seq_len[0] == ref.seq_len[0]
    wpk.wpk_destroy(plan)


def test_batch_with_inactive_slot_and_ragged_lengths():
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    model = oracle.Model(cfg, w)
    cap = 140  # 3 KV chunks, the last one partial
    lens = np.array([63, -1, 64, 129], np.int32)  # chunk edges and an inactive slot
    kc, vc = synth.synthetic_kv(cfg, 4, cap, np.maximum(lens, 0))
    tok = np.array([5, 6, 7, 999], np.int32)
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, 4, cap)
    assert plan, wpk.wpk_last_error(None)
    st = HostState(kc, vc, lens, tok, cfg.vocab)
    assert st.serial(plan, 3, poison=True) == 0
    ok_, ov_, osl = kc.copy(), vc.copy(), lens.copy()
    olog, otok = model.step(tok, ok_, ov_, osl)
    for b in (0, 2, 3):
        assert np.max(np.abs(st.logits[b] - olog[b])) < 2e-3
        assert st.tokens[b] == otok[b]
    assert st.tokens[1] == 6 and st.seq_len.tolist() == osl.tolist()
    assert np.array_equal(st.kc[:, 1], kc[:, 1])
    wpk.wpk_destroy(plan)


def test_full_cache_and_bad_token_are_errors():
    cfg, w, model, kc, vc, sl, tok = _tiny_setup(prompt_len=4, cap=4)
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, 1, 4)
    st = HostState(kc, vc, sl, tok, cfg.vocab)
    assert st.serial(plan, 0) == wpk.WPK_E_CTX_FULL
    cfg, w, model, kc, vc, sl, tok = _tiny_setup(prompt_len=4, cap=8)
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, 1, 8)
    st = HostState(kc, vc, sl, np.array([cfg.vocab + 5], np.int32), cfg.vocab)
    assert st.serial(plan, 0) == wpk.WPK_E_TOKEN


@pytest.mark.parametrize("batch", [8, 32])
def test_wide_batch_plan_matches_oracle(batch):
    """Batches above four use the matrix-core layout: norm tiles write hi/lo
    bf16 operand rows; every projection tile covers 64 weight rows and a
    512-column K slice for all sequences, and the last slice of a row block
    adds the partial sums in slice order.  The serial executor and the
    threaded protocol emulator of that DAG against the oracle, with ragged
    lengths, an inactive slot and NaN poison."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    model = oracle.Model(cfg, w)
    cap = 140
    rng = np.random.default_rng(batch)
    lens = rng.integers(1, cap - 1, size=batch).astype(np.int32)
    lens[0], lens[-1] = 63, 129
    lens[1] = -1
    kc, vc = synth.synthetic_kv(cfg, batch, cap, np.maximum(lens, 0))
    tok = rng.integers(0, cfg.vocab, size=batch).astype(np.int32)
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, batch, cap)
    assert plan, wpk.wpk_last_error(None)
    info = wpk.wpk_get_info(plan)
    assert info.rows_per_tile_h == 64 and info.rows_per_tile_f == 64
    ty, _, wait, signal = wpk.wpk_get_dag(plan, info.n_tiles)
    # layer 0's embedding rows; later RMSNorms live in the producing and consuming epilogues
    assert np.sum(np.array(ty) == 8) == batch and not np.isin(np.array(ty), [9, 10]).any()
    ok_, ov_, osl = kc.copy(), vc.copy(), lens.copy()
    olog, otok = model.step(tok, ok_, ov_, osl)
    ref = None
    for seed in (0, 5):
        st = HostState(kc, vc, lens, tok, cfg.vocab)
        assert st.serial(plan, seed, poison=True) == 0, wpk.wpk_last_error(plan)
        rc, log = wpk.wpk_get_log(plan, info.n_tiles)
        check_log(log, wait, signal)
        if ref is None:
            ref = st
        else:
            assert np.array_equal(st.logits, ref.logits)
    st = HostState(kc, vc, lens, tok, cfg.vocab)
    assert st.emulate(plan, 9, 2) == 0, wpk.wpk_last_error(plan)
    rc, log = wpk.wpk_get_log(plan, info.n_tiles)
    check_log(log, wait, signal)
    assert np.array_equal(st.logits, ref.logits)  # slice sums in a fixed order
    st = ref
    act = [b for b in range(batch) if lens[b] >= 0]
    for b in act:
        err = np.max(np.abs(st.logits[b] - olog[b]))
        assert err < 1e-3, (b, err)  # hi/lo operands keep about 16 significant bits
        top2 = np.sort(olog[b])[-2:]
        if top2[1] - top2[0] > 4e-2:
            assert st.tokens[b] == otok[b]
    assert st.tokens[1] == tok[1] and st.seq_len.tolist() == osl.tolist()
    assert np.array_equal(st.kc[:, 1], kc[:, 1])
    wpk.wpk_destroy(plan)


def test_llama_1b_batch32_dag_shape():
    """Wide Llama-1B plan: 64-row x 512-column tiles, the same tile counts per
    operator as the batch-1 plan, an embedding-row tile per sequence before
    layer 0 and no other norm tiles, and per-slice dependencies of o-proj and
    down."""
    info, (ty, layer, wait, signal) = _info_and_dag(synth.LLAMA_1B, 32, 1088)
    ty = np.array(ty)
    per_layer = {0: 192, 3: 128, 4: 1024, 5: 512}
    for t, n in per_layer.items():
        assert np.sum(ty == t) == 16 * n, t
    assert np.sum(ty == 8) == 32 and np.sum(ty == 9) == 0 and np.sum(ty == 10) == 0
    # QKV of layer l > 0 waits on the down tiles of layer l - 1 (no norm tile between)
    wait_a, sig_a, lay_a = np.array(wait), np.array(signal), np.array(layer)
    qkv1 = np.nonzero((ty == 0) & (lay_a == 1))[0]
    down0 = np.nonzero((ty == 5) & (lay_a == 0))[0]
    assert set(wait_a[qkv1].tolist()) == set(sig_a[down0].tolist())
    assert np.sum(ty == 1) == 16 * 32 * 8 * 5  # attention: 4-chunk groups of the 17 chunks
    assert np.sum(ty == 2) == 16 * 32 * 8
    # with LDS forwarding: one chained tile per (sequence, kv head), no combine tiles
    info, (ty2, _, _, _) = _info_and_dag(synth.LLAMA_1B, 32, 1088, forward=1)
    ty2 = np.array(ty2)
    assert np.sum(ty2 == 11) == 16 * 32 * 8 and np.sum(ty2 == 1) == 0 and np.sum(ty2 == 2) == 0
    assert np.sum(ty == 6) == 8016 and np.sum(ty == 7) == 1
    # down slice c waits only on the gate/up row blocks of its K slice
    wait = np.array(wait)
    down = np.nonzero((ty == 5) & (np.array(layer) == 0))[0]
    assert len(set(wait[down].tolist())) == 16


def test_lds_forwarding_is_refused_below_batch_5():
    d = dummy_desc(synth.MINI)
    assert not wpk.wpk_build_host(d.desc, 4, 100, wpk.wpk_build_opts(forward=1))
    assert "forwarding" in wpk.wpk_last_error(None)


@pytest.mark.parametrize("cfg_name,batch,forward", [("MINI", 8, 1), ("MINI", 32, -1), ("MINI", 32, 1)])
def test_lds_forwarded_attention_matches_split_attention(cfg_name, batch, forward):
    """Chained attention tiles (every KV chunk of one sequence and kv head on
    one worker, partials merged on chip, no combine tiles) against the oracle,
    and the DAG they make: one tile per (sequence, kv head), no combine tiles."""
    cfg = getattr(synth, cfg_name)
    w = synth.make_weights(cfg, gain_std=0.1)
    model = oracle.Model(cfg, w)
    cap = 140
    rng = np.random.default_rng(batch + 7)
    lens = rng.integers(1, cap - 2, size=batch).astype(np.int32)
    if batch > 1:
        lens[1] = -1
    kc, vc = synth.synthetic_kv(cfg, batch, cap, np.maximum(lens, 0))
    tok = rng.integers(0, cfg.vocab, size=batch).astype(np.int32)
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, batch, cap, wpk.wpk_build_opts(forward=forward))
    assert plan, wpk.wpk_last_error(None)
    info = wpk.wpk_get_info(plan)
    ty, _, wait, signal = wpk.wpk_get_dag(plan, info.n_tiles)
    ty = np.array(ty)
    if forward == 1:
        assert np.sum(ty == 11) == cfg.n_layers * batch * cfg.n_kv_heads
        assert np.sum(ty == 1) == 0 and np.sum(ty == 2) == 0
    else:
        assert np.sum(ty == 11) == 0 and np.sum(ty == 2) == cfg.n_layers * batch * cfg.n_kv_heads
    st = HostState(kc, vc, lens, tok, cfg.vocab)
    assert st.serial(plan, 5, poison=True) == 0, wpk.wpk_last_error(plan)
    rc, log = wpk.wpk_get_log(plan, info.n_tiles)
    check_log(log, wait, signal)
    olog, otok = model.step(tok, kc.copy(), vc.copy(), lens.copy())
    act = lens >= 0
    assert np.max(np.abs(st.logits[act] - olog[act])) < 1e-3
    assert np.array_equal(st.tokens[act], otok[act])
    wpk.wpk_destroy(plan)


@pytest.mark.parametrize("batch", [1, 8])
def test_barrier_edge_ablation_same_results_and_coarser_groups(batch):
    """The barrier-edge ablation (every consumer waits for its whole producing
    operator) builds a valid DAG with fewer, larger counter groups, and the
    serial executor gives bit-identical results to the tile-edge DAG."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    cap = 140
    lens = np.array([63, 100, 7, 128, 1, 64, 65, 90][:batch], np.int32)
    kc, vc = synth.synthetic_kv(cfg, batch, cap, lens)
    tok = (np.arange(batch, dtype=np.int32) * 113 + 5) % cfg.vocab
    d = host_desc(cfg, w)
    outs = []
    for be in (0, 1):
        plan = wpk.wpk_build_host(d.desc, batch, cap, wpk.wpk_build_opts(barrier_edges=be))
        assert plan, wpk.wpk_last_error(None)
        info = wpk.wpk_get_info(plan)
        _, _, wait, signal = wpk.wpk_get_dag(plan, info.n_tiles)
        outs.append((info, HostState(kc, vc, lens, tok, cfg.vocab)))
        assert outs[-1][1].serial(plan, 3, poison=True) == 0, wpk.wpk_last_error(plan)
        rc, log = wpk.wpk_get_log(plan, info.n_tiles)
        check_log(log, wait, signal)
        wpk.wpk_destroy(plan)
    (i0, s0), (i1, s1) = outs
    assert i1.n_tiles == i0.n_tiles and i1.n_groups < i0.n_groups
    assert np.array_equal(s0.logits, s1.logits) and np.array_equal(s0.kc, s1.kc)


def test_emulated_fixed_reducer_matches_serial_on_a_matrix_core_plan():
    """The fixed-reducer scheme (each wide row block reduced by its last slice
    in claim order, which waits for its siblings) through the C ABI's host
    emulator: bitwise equal to the serial executor, every tile once; device
    plans do not offer it."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    batch, cap = 8, 140
    lens = np.array([63, 100, 7, 128, 1, 64, 65, -1], np.int32)
    kc, vc = synth.synthetic_kv(cfg, batch, cap, np.maximum(lens, 0))
    tok = (np.arange(batch, dtype=np.int32) * 113 + 5) % cfg.vocab
    d = host_desc(cfg, w)
    plan = wpk.wpk_build_host(d.desc, batch, cap)
    n = wpk.wpk_get_info(plan).n_tiles
    _, _, wait, signal = wpk.wpk_get_dag(plan, n)
    ref = HostState(kc, vc, lens, tok, cfg.vocab)
    assert ref.serial(plan, 5) == 0
    assert wpk.wpk_set_option(plan, wpk.WPK_OPT_FIXED_REDUCER, 1) == 0
    for seed in (1, 2):
        st = HostState(kc, vc, lens, tok, cfg.vocab)
        assert st.emulate(plan, 16, seed) == 0, wpk.wpk_last_error(plan)
        rc, log = wpk.wpk_get_log(plan, n)
        check_log(log, wait, signal, canonical_only=True)
        assert np.array_equal(st.logits, ref.logits) and np.array_equal(st.kc, ref.kc)
    assert wpk.wpk_set_option(plan, wpk.WPK_OPT_FIXED_REDUCER, 2) == wpk.WPK_E_ARG
    wpk.wpk_destroy(plan)


@pytest.mark.parametrize("batch", [1, 8])
def test_split_plan_emulated_matches_serial(batch):
    """A plan split into two co-resident megakernels (attention and combine
    tiles in their own claim queues) runs on the emulator's workers to the
    serial executor's results bit for bit, with a valid log; a negative worker
    count is refused."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    cap = 140
    lens = np.array([63, 100, 7, 128, 1, 64, 65, 90][:batch], np.int32)
    kc, vc = synth.synthetic_kv(cfg, batch, cap, lens)
    tok = (np.arange(batch, dtype=np.int32) * 113 + 5) % cfg.vocab
    d = host_desc(cfg, w)
    assert not wpk.wpk_build_host(d.desc, batch, cap, wpk.wpk_build_opts(split_workers=-1))
    plan = wpk.wpk_build_host(d.desc, batch, cap, wpk.wpk_build_opts(split_workers=64))
    assert plan, wpk.wpk_last_error(None)
    info = wpk.wpk_get_info(plan)
    _, _, wait, signal = wpk.wpk_get_dag(plan, info.n_tiles)
    ref = HostState(kc, vc, lens, tok, cfg.vocab)
    assert ref.serial(plan, 1, poison=True) == 0, wpk.wpk_last_error(plan)
    st = HostState(kc, vc, lens, tok, cfg.vocab)
    assert st.emulate(plan, 16, 7) == 0, wpk.wpk_last_error(plan)
    rc, log = wpk.wpk_get_log(plan, info.n_tiles)
    check_log(log, wait, signal)
    assert np.array_equal(st.logits, ref.logits) and np.array_equal(st.kc, ref.kc)
    # 8 claim queues per megakernel: fewer than 16 emulated workers is refused
    assert HostState(kc, vc, lens, tok, cfg.vocab).emulate(plan, 8, 7) != 0
    wpk.wpk_destroy(plan)
