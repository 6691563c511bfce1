"""GPU parity of the prompt prefill (time to first token) against the CPU
oracle, whose prefill is its decode step run token by token over the prompt
(teacher-forced): the same causal computation.

Bars: logits of the last prompt position max |error| <= 2e-2 (bf16 weights),
the first generated token identical up to reported near ties, the KV cache
of every prompt position within a few bf16 steps of the oracle's (the
prefill rounds activations to bf16 at each matrix product; the oracle keeps
them in fp64), seq_len = prompt length, every tile run once after its
producers (per-tile log).  The three executions -- one megakernel, two
co-resident megakernels, the per-operator hipGraph -- share the tile bodies
and must agree bitwise.  At the full Llama-3.2-1B shape and a 496-token
prompt at batch 16 the oracle's token-by-token prefill would take minutes,
so there the K/V of sampled layer-0 positions are compared with the oracle's
own RMSNorm, matvec and RoPE, and the rest is checked by properties.
"""
import numpy as np
import pytest
import torch

import oracle
import persistent_megakernel_latency_amd as wpk
import synth
from tests.gpu_helpers import announce, from_dev, to_dev, tokens_agree
from tests.helpers import check_log

pytestmark = pytest.mark.gpu


class Prefill:
    def __init__(self, cfg, w, batch, cap, prompt_len, mode=0, split_workers=0, desc=None, fill=0):
        self.cfg = cfg
        if desc is None:
            desc, self.tensors = wpk.model_from_weights(cfg, w, "cuda")
        self.desc = desc
        opts = wpk.wpk_prefill_opts(mode=mode, split_workers=split_workers)
        self.plan = wpk.wpk_build_prefill(desc.desc, batch, cap, prompt_len, opts)
        assert self.plan, wpk.wpk_prefill_last_error(None)
        self.info = wpk.wpk_prefill_get_info(self.plan)
        shape = (cfg.n_layers, batch, cfg.n_kv_heads, cap, cfg.head_dim)
        self.kc = torch.full(shape, fill, dtype=torch.int16, device="cuda")
        self.vc = torch.full(shape, fill, dtype=torch.int16, device="cuda")
        self.seq = torch.full((batch,), -5, dtype=torch.int32, device="cuda")
        self.logits = torch.zeros((batch, cfg.vocab), dtype=torch.float32, device="cuda")
        self.tok = torch.full((batch,), -1, dtype=torch.int32, device="cuda")
        self.kv = wpk.wpk_kv(self.kc.data_ptr(), self.vc.data_ptr(), self.seq.data_ptr())

    def run(self, prompt: np.ndarray):
        p = torch.from_numpy(np.ascontiguousarray(prompt, np.int32)).cuda()
        wpk.check_prefill(wpk.wpk_prefill(self.plan, p.data_ptr(), self.kv, self.logits.data_ptr(),
                                          self.tok.data_ptr(), 0), self.plan, "wpk_prefill")
        wpk.check_prefill(wpk.wpk_prefill_sync(self.plan), self.plan, "wpk_prefill_sync")
        return (self.kc.cpu().numpy().view(np.uint16), self.vc.cpu().numpy().view(np.uint16),
                self.seq.cpu().numpy(), self.tok.cpu().numpy(), self.logits.cpu().numpy())

    def log(self):
        rc, log = wpk.wpk_prefill_get_log(self.plan, self.info.n_tiles)
        wpk.check_prefill(rc, self.plan, "wpk_prefill_get_log")
        return log

    def dag(self):
        return wpk.wpk_prefill_get_dag(self.plan, self.info.n_tiles)

    def close(self):
        if self.plan:
            wpk.wpk_prefill_destroy(self.plan)
            self.plan = None


def _bf16(a):
    return (a.astype(np.uint32) << 16).view(np.float32)


def _compare(cfg, w, batch, cap, prompt_len, seed, log=True, kv_tol=3e-2, fill=0):
    """fill: the cache's initial 16-bit pattern (0, or a NaN whose rows past
    the prompt must come back unchanged)."""
    prompt = synth.prompt_tokens(cfg, batch, prompt_len, seed=seed)
    model = oracle.Model(cfg, w)
    okc, ovc = model.new_cache(batch, cap)
    osl = np.zeros(batch, np.int32)
    announce(f"prefill {cfg.name} b{batch} P{prompt_len}: oracle")
    olog, otok = model.prefill(prompt, okc, ovc, osl)
    announce(f"prefill {cfg.name} b{batch} P{prompt_len}: build")
    g = Prefill(cfg, w, batch, cap, prompt_len, fill=fill)
    try:
        if log:
            wpk.check_prefill(wpk.wpk_prefill_set_option(g.plan, wpk.WPK_OPT_LOG, 1), g.plan)
        announce(f"prefill {cfg.name} b{batch} P{prompt_len}: run")
        kc, vc, sl, tok, lg = g.run(prompt)
        assert np.all(sl == prompt_len)
        worst = 0.0
        for b in range(batch):
            err = float(np.max(np.abs(lg[b] - olog[b])))
            worst = max(worst, err)
            assert err <= 2e-2, f"seq {b}: max |logit err| {err}"
            ok, why = tokens_agree(int(tok[b]), int(otok[b]), olog[b], err)
            assert ok, f"seq {b}: {why}"
        for name, got, want in (("K", kc, okc), ("V", vc, ovc)):
            d = np.abs(_bf16(got[:, :, :, :prompt_len]) - _bf16(want[:, :, :, :prompt_len]))
            assert float(d.max()) <= kv_tol, f"{name} cache: max |err| {float(d.max())}"
            assert float(d.mean()) <= kv_tol / 10, f"{name} cache: mean |err| {float(d.mean())}"
            # positions past the prompt untouched
            assert np.all(got[:, :, :, prompt_len:] == np.uint16(fill & 0xFFFF)), f"{name} cache written past the prompt"
        if log:
            ty, layer, wait, signal, queue = g.dag()
            check_log(g.log(), wait, signal)
        return worst
    finally:
        g.close()


@pytest.mark.parametrize("batch,prompt_len,cap", [(3, 150, 200), (1, 1, 64), (5, 128, 160), (2, 257, 300)])
def test_mini_prefill_matches_oracle(batch, prompt_len, cap):
    """Several row blocks with a ragged tail (150, 257), exactly one block
    (128), a single token (1)."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    _compare(cfg, w, batch, cap, prompt_len, seed=7 + prompt_len)


def test_mini_prefill_over_a_nan_filled_cache():
    """The cache starts as NaN bit patterns: the prefill reads no cache row it
    has not written (attention keys stay inside the prompt), so logits and
    tokens match the oracle and rows past the prompt keep their bits."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    _compare(cfg, w, 3, 200, 150, seed=41, fill=0x7FC0)


def test_llama_prefill_short_prompt_matches_oracle():
    """All 16 layers at the full Llama-3.2-1B width, a 40-token prompt."""
    cfg = synth.LLAMA_1B
    w = synth.make_weights(cfg, gain_std=0.1)
    _compare(cfg, w, 2, 64, 40, seed=21, log=True, kv_tol=5e-2)


def _modes_agree(cfg, w, batch, cap, prompt_len, seed):
    prompt = synth.prompt_tokens(cfg, batch, prompt_len, seed=seed)
    first = None
    desc, tensors = wpk.model_from_weights(cfg, w, "cuda")
    for mode in (wpk.WPK_PREFILL_MEGAKERNEL, wpk.WPK_PREFILL_SPLIT, wpk.WPK_PREFILL_GRAPH):
        g = Prefill(cfg, w, batch, cap, prompt_len, mode=mode, desc=desc)
        try:
            for rep in range(2):  # a second run on the same plan (epochs, argmax shards reset)
                announce(f"prefill {cfg.name} b{batch} P{prompt_len} mode {mode} run {rep}")
                out = g.run(prompt)
                if first is None:
                    first = out
                    continue
                for name, a, b in zip(("K", "V", "seq_len", "token", "logits"), first, out):
                    assert np.array_equal(a, b), f"mode {mode} run {rep}: {name} differs"
        finally:
            g.close()
    return first


def test_mini_prefill_modes_bitwise():
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    _modes_agree(cfg, w, 4, 200, 150, seed=5)


def test_llama_ttft_config_sampled():
    """The time-to-first-token workload: Llama-3.2-1B shape, batch 16, a
    496-token prompt.  The three executions agree bitwise; layer-0 K and V of
    sampled positions match the oracle's RMSNorm, matvec and RoPE; every
    first token is the greedy choice of its logits (lowest index on ties);
    the per-tile log is canonical."""
    cfg = synth.LLAMA_1B
    w = synth.make_weights(cfg, gain_std=0.1)
    batch, cap, P = 16, 512, 496
    kc, vc, sl, tok, lg = _modes_agree(cfg, w, batch, cap, P, seed=4)
    assert np.all(sl == P)
    assert np.all(np.isfinite(lg))
    for b in range(batch):
        assert int(tok[b]) == oracle.argmax_f32(lg[b].astype(np.float64))
    prompt = synth.prompt_tokens(cfg, batch, P, seed=4)
    emb = _bf16(w["embed"])
    lw = w["layers"][0]
    d, hq, hkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    rng = np.random.default_rng(3)
    worst = 0.0
    for b, p in [(0, 0), (15, P - 1), (7, 255), (3, 256)] + [(int(x), int(y)) for x, y in
                                                             zip(rng.integers(0, batch, 6), rng.integers(0, P, 6))]:
        x = emb[prompt[b, p]].astype(np.float64)
        y = oracle.rmsnorm(x, lw["attn_norm"], cfg.rms_eps)
        kv = oracle.matvec(lw["w_qkv"][hq * d:], y, oracle.BF16)
        for g in range(hkv):
            k = oracle.rope(kv[g * d:(g + 1) * d], p, cfg.rope_theta)
            v = kv[(hkv + g) * d:(hkv + g + 1) * d]
            worst = max(worst, float(np.max(np.abs(_bf16(kc[0, b, g, p]) - k))),
                        float(np.max(np.abs(_bf16(vc[0, b, g, p]) - v))))
    assert worst <= 3e-2, f"layer-0 K/V max |err| {worst}"
    announce("prefill llama b16 P496: logged run")
    g = Prefill(cfg, w, batch, cap, P)
    try:
        wpk.check_prefill(wpk.wpk_prefill_set_option(g.plan, wpk.WPK_OPT_LOG, 1), g.plan)
        out = g.run(prompt)
        for a, b2 in zip(out, (kc, vc, sl, tok, lg)):
            assert np.array_equal(a, b2)
        ty, layer, wait, signal, queue = g.dag()
        check_log(g.log(), wait, signal)
    finally:
        g.close()


def test_prefill_then_decode_step():
    """The prefill's cache and first token feed the decode step directly: one
    decode step after the prefill matches the oracle's step after its own
    prefill (MINI, batch 8: the matrix-core decode plan)."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    batch, cap, P = 8, 200, 100
    prompt = synth.prompt_tokens(cfg, batch, P, seed=9)
    model = oracle.Model(cfg, w)
    okc, ovc = model.new_cache(batch, cap)
    osl = np.zeros(batch, np.int32)
    _, otok = model.prefill(prompt, okc, ovc, osl)
    desc, tensors = wpk.model_from_weights(cfg, w, "cuda")
    announce("prefill then decode: prefill")
    g = Prefill(cfg, w, batch, cap, P, desc=desc)
    try:
        kc, vc, sl, tok, lg = g.run(prompt)
        # continue both from the GPU's state (the prefill's own rounding is covered above)
        okc2, ovc2, osl2 = kc.copy(), vc.copy(), sl.copy()
        olog, otok2 = model.step(tok, okc2, ovc2, osl2)
        plan = wpk.wpk_build(desc.desc, batch, cap)
        assert plan, wpk.wpk_last_error(None)
        try:
            announce("prefill then decode: decode step")
            wpk.check(wpk.wpk_step(plan, g.tok.data_ptr(), g.kv, g.logits.data_ptr(), 0), plan, "wpk_step")
            wpk.check(wpk.wpk_sync(plan), plan, "wpk_sync")
            dlog = g.logits.cpu().numpy()
            dtok = g.tok.cpu().numpy()
            assert np.array_equal(g.seq.cpu().numpy(), np.full(batch, P + 1))
            for b in range(batch):
                err = float(np.max(np.abs(dlog[b] - olog[b])))
                assert err <= 2e-2, f"seq {b}: {err}"
                ok, why = tokens_agree(int(dtok[b]), int(otok2[b]), olog[b], err)
                assert ok, why
        finally:
            wpk.wpk_destroy(plan)
    finally:
        g.close()


def test_prefill_bad_token_latches():
    cfg = synth.MINI
    w = synth.make_weights(cfg)
    g = Prefill(cfg, w, 2, 64, 10)
    try:
        prompt = synth.prompt_tokens(cfg, 2, 10, seed=1)
        prompt[1, 3] = cfg.vocab  # out of range
        p = torch.from_numpy(prompt.astype(np.int32)).cuda()
        announce("prefill bad token")
        wpk.check_prefill(wpk.wpk_prefill(g.plan, p.data_ptr(), g.kv, g.logits.data_ptr(), g.tok.data_ptr(), 0),
                          g.plan)
        assert wpk.wpk_prefill_sync(g.plan) == wpk.WPK_E_TOKEN
        assert wpk.wpk_prefill(g.plan, p.data_ptr(), g.kv, g.logits.data_ptr(), g.tok.data_ptr(), 0) == \
            wpk.WPK_E_STATE
        wpk.check_prefill(wpk.wpk_prefill_set_option(g.plan, wpk.WPK_OPT_RESET, 1), g.plan)
        prompt[1, 3] = 5
        g.run(prompt)
    finally:
        g.close()


def test_prefill_refuses_weights_outside_the_fp16_range():
    """The o-projection, gate/up and down products run in fp16: a down
    weight of ~1e5 cannot be converted, and the build says so."""
    cfg = synth.MINI
    w = synth.make_weights(cfg)
    w["layers"][1]["w_down"][5, 7] = np.uint16(0x47C3)  # bf16 99840
    desc, tensors = wpk.model_from_weights(cfg, w, "cuda")
    announce("prefill fp16 weight range")
    plan = wpk.wpk_build_prefill(desc.desc, 2, 64, 10, None)
    assert not plan
    assert "fp16" in wpk.wpk_prefill_last_error(None)
    w["layers"][1]["w_down"][5, 7] = np.uint16(0x477F)  # bf16 65280: inside the range
    desc, tensors = wpk.model_from_weights(cfg, w, "cuda")
    plan = wpk.wpk_build_prefill(desc.desc, 2, 64, 10, None)
    assert plan, wpk.wpk_prefill_last_error(None)
    wpk.wpk_prefill_destroy(plan)


def test_prefill_fp16_activation_overflow_latches():
    """An MLP RMSNorm gain of 1e5 drives the gate/up operand past the fp16
    range: the norm tile latches WPK_E_RANGE (every worker then leaves through
    the abort flag), the plan refuses to run until reset, and runs again
    after it (latching the same error: the gains are the caller's)."""
    cfg = synth.MINI
    w = synth.make_weights(cfg)
    w["layers"][0]["mlp_norm"][:] = np.float32(1e5)
    g = Prefill(cfg, w, 2, 64, 10)
    try:
        prompt = synth.prompt_tokens(cfg, 2, 10, seed=3)
        p = torch.from_numpy(prompt.astype(np.int32)).cuda()
        announce("prefill fp16 activation overflow")
        for _ in range(2):
            wpk.check_prefill(wpk.wpk_prefill(g.plan, p.data_ptr(), g.kv, g.logits.data_ptr(), g.tok.data_ptr(), 0),
                              g.plan)
            assert wpk.wpk_prefill_sync(g.plan) == wpk.WPK_E_RANGE
            assert wpk.wpk_prefill(g.plan, p.data_ptr(), g.kv, g.logits.data_ptr(), g.tok.data_ptr(), 0) == \
                wpk.WPK_E_STATE
            wpk.check_prefill(wpk.wpk_prefill_set_option(g.plan, wpk.WPK_OPT_RESET, 1), g.plan)
    finally:
        g.close()


def test_split_prefill_log_places_attention_in_its_pool():
    """Two co-resident megakernels: the canonical log holds, and the attention
    tiles -- and only they -- ran on the last split_workers workers."""
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    batch, cap, P, w1 = 3, 200, 150, 64
    prompt = synth.prompt_tokens(cfg, batch, P, seed=13)
    announce("prefill split log")
    g = Prefill(cfg, w, batch, cap, P, mode=wpk.WPK_PREFILL_SPLIT, split_workers=w1)
    try:
        assert g.info.split_workers == w1
        wpk.check_prefill(wpk.wpk_prefill_set_option(g.plan, wpk.WPK_OPT_LOG, 1), g.plan)
        g.run(prompt)
        ty, layer, wait, signal, queue = g.dag()
        log = g.log()
        check_log(log, wait, signal)
        from tests.helpers import log_array
        a = log_array(log)
        w0 = g.info.workers - w1
        attn = np.asarray(ty) == wpk.PREFILL_TILE_TYPES.index("attn")
        assert np.all(a["worker"][attn] >= w0)
        assert np.all(a["worker"][~attn] < w0)
    finally:
        g.close()
