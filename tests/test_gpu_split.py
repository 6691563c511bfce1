"""Two co-resident megakernels (wpk_build_opts.split_workers): the attention and
combine tiles claimed only by the launch's last split_workers workers, every
other tile only by the others, both synchronised through the same counters.

The split changes which worker runs a tile, not what a tile computes, so a
split plan must equal the single megakernel bitwise, step after step; its
logged steps must pass the canonical log check and show every attention and
combine tile run by the second megakernel's workers and no other tile."""
import numpy as np
import pytest

import persistent_megakernel_latency_amd as wpk
import synth
from tests.gpu_helpers import GpuPlan, announce
from tests.helpers import check_log, log_array

pytestmark = pytest.mark.gpu


def _case(batch, cap, seed):
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, cap - 8, size=batch).astype(np.int32)
    lens[0] = 63
    kc, vc = synth.synthetic_kv(cfg, batch, cap, lens)
    tok = rng.integers(0, cfg.vocab, size=batch).astype(np.int32)
    return cfg, w, kc, vc, lens, tok


@pytest.mark.parametrize("batch,split,coop", [(3, 128, 0), (32, 128, 0), (32, 100, 1)])
def test_split_equals_single_megakernel_bitwise(batch, split, coop):
    cap = 140
    cfg, w, kc, vc, lens, tok = _case(batch, cap, seed=5 + batch)
    announce(f"split b{batch} w1={split} build")
    a = GpuPlan(cfg, w, batch, cap, kc, vc, lens, tok)
    b = GpuPlan(cfg, w, batch, cap, kc, vc, lens, tok, desc=a.desc, opts=wpk.wpk_build_opts(split_workers=split))
    if coop:
        wpk.check(wpk.wpk_set_option(b.plan, wpk.WPK_OPT_LAUNCH, 1), b.plan)
    ty, layer, wait, signal = b.dag()
    for s in range(3):
        announce(f"split b{batch} w1={split} step {s}")
        wpk.check(wpk.wpk_set_option(b.plan, wpk.WPK_OPT_LOG, 1 if s == 1 else 0), b.plan)
        a.step()
        b.step()
        for x, y in zip(a.state(), b.state()):
            assert np.array_equal(x, y), f"step {s}"
        if s == 1:
            check_log(b.log(), wait, signal)
            w0 = b.info.workers - split
            # attention and combine tiles ran only in the second megakernel
            ran_by = log_array(b.log())["worker"][: b.info.n_tiles]
            is_attn = np.isin(np.asarray(ty), [1, 2, 11])
            assert np.all((ran_by >= w0) == is_attn)
    a.close()
    b.close()


def test_split_refusals():
    cfg, w, kc, vc, lens, tok = _case(3, 140, seed=1)
    announce("split refusals")
    desc, keep = wpk.model_from_weights(cfg, w, "cuda")
    for bad in (-1, 4, 508, 4096):
        p = wpk.wpk_build_ex(desc.desc, 3, 140, wpk.wpk_build_opts(split_workers=bad))
        assert not p, f"split_workers={bad} accepted"
    g = GpuPlan(cfg, w, 3, 140, kc, vc, lens, tok, desc=desc, opts=wpk.wpk_build_opts(split_workers=64))
    assert wpk.wpk_set_option(g.plan, wpk.WPK_OPT_WORKERS, 256) == wpk.WPK_E_ARG
    rc = wpk.wpk_persist_begin(g.plan, g.tokens.data_ptr(), g.kv, g.logits.data_ptr(), 0)
    assert rc == wpk.WPK_E_ARG
    g.step()
    g.close()
