"""The allocation-free entry point: a plan whose workspace is the library's
static device array (wpk_build_static) against the same plan built with its
own allocation (wpk_build), through the C ABI, on two builds in a row (the
second smaller); the array's ownership rule; and the size limit."""
import numpy as np
import pytest

import persistent_megakernel_latency_amd as wpk
import synth
from tests.gpu_helpers import GpuPlan, announce
from tests.helpers import dummy_desc

pytestmark = pytest.mark.gpu


def _pair(cfg, batch, cap, lens, tok, gain_std=0.1):
    w = synth.make_weights(cfg, gain_std=gain_std)
    kc, vc = synth.synthetic_kv(cfg, batch, cap, lens)
    ref = GpuPlan(cfg, w, batch, cap, kc, vc, lens, tok)
    stat = GpuPlan(cfg, w, batch, cap, kc, vc, lens, tok, desc=ref.desc, static=True)
    return ref, stat


def _same_steps(ref, stat, steps, name):
    for s in range(steps):
        announce(f"no-alloc {name} step {s}")
        ref.step()
        stat.step()
        for x, y in zip(ref.state(), stat.state()):
            assert np.array_equal(x, y), f"{name} step {s}"


def test_static_workspace_matches_allocated_plan_on_two_builds():
    # first build: MINI (bf16), three sequences with ragged contexts
    ref1, st1 = _pair(synth.MINI, 3, 200, np.array([63, 150, 5], np.int32), np.array([11, 500, 999], np.int32))
    assert wpk.wpk_get_info(st1.plan).workspace_bytes <= wpk.WPK_STATIC_SCRATCH_BYTES
    _same_steps(ref1, st1, 2, "mini b3")
    # second build, smaller (tiny, float32, one sequence): it takes the array
    # over and clears what must start at zero; the first static plan then
    # refuses to step
    ref2, st2 = _pair(synth.TINY, 1, 64, np.array([40], np.int32), np.array([7], np.int32))
    assert wpk.wpk_get_info(st2.plan).workspace_bytes < wpk.wpk_get_info(st1.plan).workspace_bytes
    _same_steps(ref2, st2, 2, "tiny b1")
    rc = wpk.wpk_step(st1.plan, st1.tokens.data_ptr(), st1.kv, st1.logits.data_ptr(), 0)
    assert rc == wpk.WPK_E_STATE and "later static plan" in wpk.wpk_last_error(st1.plan)
    for g in (ref1, st1, ref2, st2):
        g.close()


def test_static_workspace_refuses_a_plan_that_does_not_fit():
    d = dummy_desc(synth.LLAMA_1B)  # never dereferenced: the size check comes first
    assert not wpk.wpk_build_static(d.desc, 32, 1088)
    msg = wpk.wpk_last_error(None)
    assert "static" in msg and str(wpk.WPK_STATIC_SCRATCH_BYTES) in msg
