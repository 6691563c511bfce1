"""Pins of the CPU oracle against things other than itself.

Each building block is checked against a library routine, a closed form, an
invariant or brute force, chosen so that a dropped term, a wrong sign, a wrong
index or a transposed operand fails at least one test.  The whole model is
pinned against a dense float64 torch forward (tests/dense_ref.py).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from tests.dense_ref import dense_logits, round_bf16_via_f32, round_f32

RNG = np.random.default_rng(12345)


# ---- number formats --------------------------------------------------------------

def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def test_round_bf16_matches_torch_on_float32_values():
    vals = [RNG.standard_normal(4000).astype(np.float32) * 10.0 ** RNG.integers(-40, 38, 4000)]
    # exact ties: float32 values whose low 16 bits are 0x8000 (both parities)
    u = (RNG.integers(0, 2 ** 31, 2000, dtype=np.uint64) & 0x7FFF0000) | 0x8000
    vals.append(u.astype(np.uint32).view(np.float32))
    vals.append(np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40, -1e-40, 1e-45, 65504.0,
                          np.float32(1.0 + 2.0 ** -8), np.float32(1.0 + 3 * 2.0 ** -8)], np.float32))
    x = np.concatenate(vals)
    x = x[np.isfinite(x)]
    want = _torch_bf16_bits(x)
    got = np.array([oracle.round_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_round_bf16_on_float64_values_off_the_float32_grid():
    """Rounding straight from float64 to bf16, with expected bits from the
    definition (8 significant bits, nearest, ties to even).  Inputs sit
    between float32 values, so rounding through float32 first (a double
    rounding) fails: 1 + 2^-8 + 2^-30 is above the halfway point between the
    bf16 neighbours 1 and 1 + 2^-7, but its float32 rounding is the exact tie
    1 + 2^-8, which goes to even (1.0)."""
    e = 2.0 ** -8  # half a bf16 ulp at 1
    cases = [
        (1.0 + e, 0x3F80),                    # exact tie: to even (1.0)
        (1.0 + 3 * e, 0x3F82),                # exact tie: to even (1 + 2^-6)
        (1.0 + e + 2.0 ** -40, 0x3F81),       # just above the tie: up
        (1.0 + e + 2.0 ** -30, 0x3F81),       # above the tie, float32 rounds it onto the tie
        (1.0 + e - 2.0 ** -40, 0x3F80),       # just below the tie: down
        (1.0 + 3 * e - 2.0 ** -40, 0x3F81),   # below an odd-side tie: down to odd
        (-(1.0 + e + 2.0 ** -40), 0xBF81),    # the sign is kept
        (3.0 + 2.0 ** -7 + 2.0 ** -45, 0x4041),  # [2, 4): ulp 2^-6, above the tie at 3 + 2^-7
        (2.0 ** -130 * (1 + 2.0 ** -30), 0x0001 << 3),  # subnormal: 2^-130 = 8 quanta of 2^-133
        (2.0 ** -134 + 2.0 ** -160, 0x0001),  # half a subnormal quantum and a bit: up
        (2.0 ** -134, 0x0000),                # exactly half the smallest subnormal: to even (zero)
        (2.0 ** 128 - 2.0 ** 120 + 2.0 ** 100, 0x7F7F),  # the largest bf16 plus a little: down to it
        (2.0 ** 128 - 2.0 ** 119 + 2.0 ** 100, 0x7F80),  # past the largest bf16 + half an ulp: inf
    ]
    for x, bits in cases:
        assert oracle.round_bf16(x) == bits, (x, hex(oracle.round_bf16(x)), hex(bits))
    # the double-rounding case really differs from rounding through float32
    x = 1.0 + e + 2.0 ** -30
    assert _torch_bf16_bits(np.array([x], np.float32))[0] == 0x3F80


def test_bf16_value_round_trip():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    for b in bits:
        v = oracle.bf16_value(int(b))
        if math.isnan(v):
            continue
        assert oracle.round_bf16(v) == int(b)


# ---- matvec ------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_matvec_vs_numpy_fp64(dtype):
    w = synth.normal(7, 0, (37, 129), 0.05, dtype=dtype)
    x = RNG.standard_normal(129)
    got = oracle.matvec(w, x, oracle.F32 if dtype == "f32" else oracle.BF16)
    wf = w.astype(np.float64) if dtype == "f32" else (
        (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    want = wf @ x
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)
    # transposition check: a non-square matrix against its transpose product fails
    assert got.shape == (37,)


# ---- RMSNorm --------------------------------------------------------------------------

def test_rmsnorm_vs_torch():
    x = RNG.standard_normal(300) * 3
    g = (1 + 0.1 * RNG.standard_normal(300)).astype(np.float32)
    got = oracle.rmsnorm(x, g, 1e-5)
    want = F.rms_norm(torch.from_numpy(x), (300,), weight=torch.from_numpy(g.astype(np.float64)), eps=1e-5)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-14, atol=0)


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = RNG.standard_normal(512)
    ones = np.ones(512, np.float32)
    y = oracle.rmsnorm(x, ones, 0.0)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-14
    for c in (1e-3, 7.5, 1e4):
        np.testing.assert_allclose(oracle.rmsnorm(c * x, ones, 0.0), y, rtol=1e-13)
    # eps is added inside the square root: a tiny vector is damped, not blown up
    tiny = 1e-6 * x
    yt = oracle.rmsnorm(tiny, ones, 1e-5)
    assert np.sqrt(np.mean(yt * yt)) < 0.01


# ---- RoPE ----------------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    v = RNG.standard_normal(64)
    assert np.array_equal(oracle.rope(v, 0, 500000.0), v)


def test_rope_preserves_norm_and_pairs():
    v = RNG.standard_normal(64)
    r = oracle.rope(v, 37, 500000.0)
    assert abs(np.linalg.norm(r) - np.linalg.norm(v)) < 1e-12
    # each pair (i, i+32) keeps its own norm: the rotation pairs i with i+32
    for i in range(32):
        assert abs(math.hypot(r[i], r[i + 32]) - math.hypot(v[i], v[i + 32])) < 1e-12


def test_rope_relative_position_invariance():
    q, k = RNG.standard_normal(64), RNG.standard_normal(64)
    for m, n, t in [(5, 3, 11), (100, 40, 250), (0, 7, 1000)]:
        a = oracle.rope(q, m, 500000.0) @ oracle.rope(k, n, 500000.0)
        b = oracle.rope(q, m + t, 500000.0) @ oracle.rope(k, n + t, 500000.0)
        assert abs(a - b) < 1e-11


def test_rope_closed_form_special_cases():
    # pair 0 has inverse frequency theta^0 = 1: unit vector e_0 at position p
    # goes to (cos p, sin p) in dims (0, 32) -- rotate-half pairing and the
    # direction of rotation.
    e0 = np.zeros(64)
    e0[0] = 1.0
    for p in (1, 2, 17):
        r = oracle.rope(e0, p, 500000.0)
        assert abs(r[0] - math.cos(p)) < 1e-15 and abs(r[32] - math.sin(p)) < 1e-15
        assert np.count_nonzero(np.delete(r, [0, 32])) == 0
    # theta = 10000, d = 64: pair 16 has inverse frequency 10000^(-1/2) = 0.01,
    # so position 100 rotates it by exactly 1 radian; e_48 goes to (-sin 1, cos 1).
    e48 = np.zeros(64)
    e48[48] = 1.0
    r = oracle.rope(e48, 100, 10000.0)
    assert abs(r[16] + math.sin(1.0)) < 1e-14 and abs(r[48] - math.cos(1.0)) < 1e-14
    # the last pair (31) has inverse frequency theta^(-62/64)
    e31 = np.zeros(64)
    e31[31] = 1.0
    r = oracle.rope(e31, 1000, 10000.0)
    ang = 1000 * 10000.0 ** (-62 / 64)
    assert abs(r[31] - math.cos(ang)) < 1e-13 and abs(r[63] - math.sin(ang)) < 1e-13


# ---- SiLU ----------------------------------------------------------------------------------

def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    for z in (-30.0, -2.5, -0.1, 0.3, 1.0, 4.0, 40.0):
        # sigmoid(-z) = 1 - sigmoid(z)  =>  silu(z) - silu(-z) = z
        assert abs(oracle.silu(z) - oracle.silu(-z) - z) < 1e-13
        assert abs(oracle.silu(z) - F.silu(torch.tensor(z, dtype=torch.float64)).item()) < 1e-15
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


# ---- attention -------------------------------------------------------------------------------

def _rand_cache(hkv, cap, d, dtype):
    if dtype == oracle.BF16:
        return synth.normal(11, 0, (hkv, cap, d), 0.9, dtype="bf16"), synth.normal(11, 1, (hkv, cap, d), 0.9, dtype="bf16")
    return synth.normal(11, 0, (hkv, cap, d), 0.9), synth.normal(11, 1, (hkv, cap, d), 0.9)


def _cache_f64(c, dtype):
    if dtype == oracle.BF16:
        return (c.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return c.astype(np.float64)


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_attention_vs_torch_sdpa_gqa(dtype):
    hq, hkv, d, cap, n = 8, 2, 64, 96, 71
    kc, vc = _rand_cache(hkv, cap, d, dtype)
    q = RNG.standard_normal((hq, d))
    out, probs = oracle.attention(q, kc, vc, n, dtype)
    k = torch.from_numpy(_cache_f64(kc, dtype)[:, :n])
    v = torch.from_numpy(_cache_f64(vc, dtype)[:, :n])
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], k, v, enable_gqa=True)
    np.testing.assert_allclose(out, ref[:, 0].numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(probs.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_attention_single_position_returns_v0_exactly():
    hq, hkv, d, cap = 4, 2, 64, 8
    kc, vc = _rand_cache(hkv, cap, d, oracle.BF16)
    q = RNG.standard_normal((hq, d)) * 5
    out, probs = oracle.attention(q, kc, vc, 1, oracle.BF16)
    v = _cache_f64(vc, oracle.BF16)
    for h in range(hq):
        assert np.array_equal(out[h], v[h // 2, 0])
        assert probs[h, 0] == 1.0


def test_attention_ignores_positions_beyond_n_and_gqa_equals_repeated_mha():
    hq, hkv, d, cap, n = 8, 2, 64, 64, 40
    kc, vc = _rand_cache(hkv, cap, d, oracle.F32)
    q = RNG.standard_normal((hq, d))
    out, _ = oracle.attention(q, kc, vc, n, oracle.F32)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, n:] = np.nan
    vc2[:, n:] = 1e30
    out2, _ = oracle.attention(q, kc2, vc2, n, oracle.F32)
    assert np.array_equal(out, out2)
    # grouped-query: q head h reads kv head h // (hq/hkv) == MHA on repeated K/V
    krep = np.repeat(kc, hq // hkv, axis=0)
    vrep = np.repeat(vc, hq // hkv, axis=0)
    out3, _ = oracle.attention(q, krep, vrep, n, oracle.F32)
    assert np.array_equal(out, out3)
    # and not to h % hkv (a plausible index mistake gives a different result)
    kalt = np.concatenate([kc] * (hq // hkv), axis=0)
    valt = np.concatenate([vc] * (hq // hkv), axis=0)
    out4, _ = oracle.attention(q, kalt, valt, n, oracle.F32)
    assert not np.allclose(out, out4)


# ---- argmax ----------------------------------------------------------------------------------

def test_argmax_brute_force_and_ties():
    for _ in range(50):
        x = RNG.standard_normal(1000)
        assert oracle.argmax_f32(x) == int(np.argmax(x.astype(np.float32)))
    x = np.zeros(100)
    x[[17, 42, 99]] = 3.0
    assert oracle.argmax_f32(x) == 17
    # distinct in float64, equal after rounding to float32: the lowest index wins
    y = np.zeros(10)
    y[3] = 1.0 + 2.0 ** -30
    y[7] = 1.0 + 2.0 ** -29
    assert np.float32(y[3]) == np.float32(y[7])
    assert oracle.argmax_f32(y) == 3
    assert oracle.argmax_f32(np.array([-5.0, -1.0, -1.0, -7.0])) == 1
    # -0 and +0 compare equal (the lower index wins); a NaN is never chosen
    assert oracle.argmax_f32(np.array([-1.0, -0.0, 0.0])) == 1
    assert oracle.argmax_f32(np.array([-1.0, 0.0, -0.0])) == 1
    assert oracle.argmax_f32(np.array([np.nan, -3.0, np.nan, -2.0])) == 3


# ---- whole decode step -------------------------------------------------------------------------

def _oracle_all_positions(model, tokens):
    """Teacher-forced decode of tokens [T] from an empty cache; logits [T][V]."""
    cfg = model.cfg
    kc, vc = model.new_cache(1, len(tokens) + 3)
    sl = np.zeros(1, np.int32)
    rows = []
    for t in tokens:
        lg, _ = model.step(np.array([t], np.int32), kc, vc, sl)
        rows.append(lg[0])
    return np.stack(rows), kc, vc, sl


def test_tiny_incremental_decode_equals_dense_forward():
    cfg = synth.TINY
    w = synth.make_weights(cfg, gain_std=0.1)
    model = oracle.Model(cfg, w)
    toks = synth.prompt_tokens(cfg, 1, 24)[0]
    got, kc, vc, sl = _oracle_all_positions(model, toks)
    want = dense_logits(cfg, w, toks, round_f32).numpy()
    assert np.max(np.abs(got - want)) < 1e-10
    assert sl[0] == 24
    # the cache holds the rotated keys in float32 at positions 0..23, zeros beyond
    assert np.all(kc[:, 0, :, 24:] == 0) and np.all(vc[:, 0, :, 24:] == 0)
    assert np.all(np.any(kc[:, 0, :, :24] != 0, axis=-1))


def test_mini_bf16_incremental_decode_equals_dense_forward():
    cfg = synth.MINI
    w = synth.make_weights(cfg, gain_std=0.1)
    model = oracle.Model(cfg, w)
    toks = synth.prompt_tokens(cfg, 1, 12)[0]
    got, _, _, _ = _oracle_all_positions(model, toks)
    want = dense_logits(cfg, w, toks, round_bf16_via_f32).numpy()
    # torch rounds float64 -> bf16 through float32; rare double-rounding flips of
    # one bf16 ulp in a cached k/v move logits by far less than this bound
    assert np.max(np.abs(got - want)) < 2e-4
    assert np.median(np.abs(got - want)) < 1e-9


def test_causal_mask_future_tokens_do_not_change_the_past():
    cfg = synth.TINY
    model = oracle.Model(cfg, synth.make_weights(cfg, gain_std=0.1))
    a = synth.prompt_tokens(cfg, 1, 16)[0]
    b = a.copy()
    b[10:] = (b[10:] + 123) % cfg.vocab
    la, _, _, _ = _oracle_all_positions(model, a)
    lb, _, _, _ = _oracle_all_positions(model, b)
    assert np.array_equal(la[:10], lb[:10])
    assert not np.allclose(la[10:], lb[10:])


def test_batch_step_equals_single_sequence_steps_and_inactive_slot():
    cfg = synth.MINI
    model = oracle.Model(cfg, synth.make_weights(cfg, gain_std=0.1))
    cap = 16
    lens = np.array([5, -1, 9], np.int32)
    kvk, kvv = synth.synthetic_kv(cfg, 3, cap, np.maximum(lens, 0))
    toks = np.array([3, 4, 5], np.int32)
    kb, vb, sb = kvk.copy(), kvv.copy(), lens.copy()
    lg, nt = model.step(toks, kb, vb, sb)
    assert sb.tolist() == [6, -1, 10]
    assert nt[1] == toks[1] and np.all(lg[1] == 0)
    assert np.array_equal(kb[:, 1], kvk[:, 1]) and np.array_equal(vb[:, 1], kvv[:, 1])
    for b in (0, 2):
        k1 = np.ascontiguousarray(kvk[:, b:b + 1])
        v1 = np.ascontiguousarray(kvv[:, b:b + 1])
        s1 = lens[b:b + 1].copy()
        l1, t1 = model.step(toks[b:b + 1], k1, v1, s1)
        assert np.array_equal(l1[0], lg[b]) and t1[0] == nt[b]
        assert np.array_equal(k1[:, 0], kb[:, b])
        # only position lens[b] changed in the cache
        changed = np.any(k1[:, 0] != kvk[:, b], axis=(0, 1, 3))
        assert changed.tolist() == [p == lens[b] for p in range(cap)]


def test_step_rejects_full_cache_and_bad_token():
    cfg = synth.TINY
    model = oracle.Model(cfg, synth.make_weights(cfg))
    kc, vc = model.new_cache(1, 4)
    with pytest.raises(RuntimeError):
        model.step(np.array([1], np.int32), kc, vc, np.array([4], np.int32))
    with pytest.raises(RuntimeError):
        model.step(np.array([cfg.vocab], np.int32), kc, vc, np.array([0], np.int32))
