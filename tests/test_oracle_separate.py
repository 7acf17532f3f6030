"""Pins of the separate-checkpoint mode of the oracle (CPU only).

vLLM PR "Add separate CuTeDSL ReplaySSM checkpoints" (Overview, Claims):
an FP16 recurrence checkpoint written with stochastic rounding ("SR7") and
an FP8 read checkpoint written with nearest encoding.  Readings: "SR7" =
stochastic rounding with 7 random bits per value in the usual form (the top
7 bits of the discarded fraction plus 7 random bits, rounding away from zero
on a carry); the bits come from
Philox4x32-10 keyed by a per-call 64-bit seed with counter (value / 16,
head, slot, 0).  Pinned against the generator's published known-answer
vectors, an independent numpy statement of stochastic rounding checked over
all 128 random values, and closed forms of the flush and init.
"""
import os

import numpy as np
import pytest

import synth
from tests import oracle_refs as R

HERE = os.path.dirname(__file__)


def _kat():
    rows = []
    for line in open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, k, o = (part.split() for part in line.split("|"))
        rows.append(([int(v, 16) for v in c], [int(v, 16) for v in k], [int(v, 16) for v in o]))
    return rows


@pytest.mark.parametrize("ctr,key,out", _kat())
def test_philox_known_answers(oracle, ctr, key, out):
    assert [int(v) for v in oracle.philox4x32(ctr, key, 10)] == out


def _sr_numpy(v, u):
    """Stochastic rounding fp32 -> fp16 by its definition, in numpy: lo, hi
    bracket |v| among the fp16 values (hi = 2^16 standing for infinity past
    65504), f = (|v| - lo) / (hi - lo); round away from zero iff
    floor(128 f) + u >= 128."""
    with np.errstate(all="ignore"):
        return _sr_numpy_impl(np.asarray(v, np.float32), u)


def _sr_numpy_impl(v, u):
    a = np.abs(v.astype(np.float64))
    with np.errstate(over="ignore"):
        near = a.astype(np.float16).astype(np.float64)  # nearest (ties even), may be inf
    lo = np.where(near <= a, near, np.nextafter(near.astype(np.float16), np.float16(0)).astype(np.float64))
    lo = np.where(np.isinf(lo), 65504.0, lo)
    lo = np.where(a >= 65536.0, np.inf, lo)
    hi = np.nextafter(lo.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    hi = np.where(np.isinf(hi) & np.isfinite(lo), 65536.0, hi)
    with np.errstate(invalid="ignore", divide="ignore"):
        frac = np.where(np.isfinite(lo) & (hi > lo), (a - lo) / (hi - lo), 0.0)
    up = np.floor(128.0 * frac) + u.astype(np.float64) >= 128.0
    res = np.where(up, hi, lo)
    res = np.where(res >= 65536.0, np.inf, res)
    out = (np.sign(v) * res).astype(np.float16)
    out = np.where(v == 0, v.astype(np.float16), out)  # keeps the sign of zero
    return out.view(np.uint16)


def _probe_values(rng):
    parts = [
        rng.standard_normal(4000).astype(np.float32) * 0.1,          # typical states
        (rng.standard_normal(1000) * 1e-6).astype(np.float32),       # fp16 subnormal range
        rng.uniform(6e4, 7e4, 500).astype(np.float32),               # around the largest finite value
        rng.standard_normal(500).astype(np.float32).astype(np.float16).astype(np.float32),  # exact fp16
        np.array([0.0, -0.0, 65504.0, -65504.0, 65519.0, 65536.0, 1e-9, 5.96e-8, 2.0 ** -24], np.float32),
    ]
    return np.concatenate(parts)


def test_sr_matches_definition_for_every_random_value(oracle):
    rng = np.random.default_rng(11)
    v = _probe_values(rng)
    for u in range(128):
        uu = np.full(v.shape, u, np.uint8)
        got = oracle.sr_f16(v, uu)
        want = _sr_numpy(v, uu)
        assert np.array_equal(got, want), u


def test_sr_counts_and_exact_values(oracle):
    """Over the 128 random values a value rounds away from zero exactly
    floor(128 frac) times; fp16 values never move."""
    rng = np.random.default_rng(12)
    v = (rng.standard_normal(300) * 0.5).astype(np.float32)
    all_u = np.arange(128, dtype=np.uint8)
    for x in v:
        res = np.abs(oracle.sr_f16(np.full(128, x, np.float32), all_u).view(np.float16).astype(np.float64))
        a = abs(float(x))
        near = np.float16(a)
        if float(near) == a:
            assert np.all(res == a)
            continue
        lo = near if float(near) < a else np.nextafter(near, np.float16(0))
        hi = np.nextafter(lo, np.float16(np.inf))
        lo, hi = float(lo), float(hi)
        assert np.all((res == lo) | (res == hi))
        frac = (a - lo) / (hi - lo)
        assert int(np.sum(res == hi)) == int(np.floor(128 * frac)), (x, frac)


def test_sr_special_values(oracle):
    """NaN stays a quiet NaN with its sign; values below 1/128 of the fp16
    spacing above an fp16 value never round away; 65504 < |v| < 65536 goes
    to infinity only from the top 7 bits of its fraction."""
    u = np.arange(128, dtype=np.uint8)
    nan = oracle.sr_f16(np.full(128, np.nan, np.float32), u)
    assert np.all(nan == 0x7E00)
    assert np.all(oracle.sr_f16(np.full(128, -np.nan, np.float32), u) == 0xFE00)
    tiny = np.float32(2.0 ** -24 / 256)  # 1/256 of the subnormal spacing
    assert np.all(oracle.sr_f16(np.full(128, tiny, np.float32), u) == 0)
    big = np.float32(65504.0 + 32.0 * 0.75)  # f = 3/4 between 65504 and "65536"
    got = oracle.sr_f16(np.full(128, big, np.float32), u)
    assert int(np.sum(got == 0x7C00)) == 96 and int(np.sum(got == 0x7BFF)) == 32


def test_sr_bits_come_from_philox(oracle):
    seed = 0x0123456789ABCDEF
    bits = oracle.sr_bits(seed, 5, 3, 64)
    for e in range(64):
        words = oracle.philox4x32([e // 16, 3, 5, 0], [seed & 0xFFFFFFFF, seed >> 32], 10)
        j = e % 16
        assert bits[e] == (int(words[j // 4]) >> (8 * (j % 4))) & 0x7F


def test_sr_is_unbiased_up_to_the_7_bit_resolution(oracle):
    """Mean over many seeds: lo + (hi - lo) floor(128 frac) / 128."""
    x = np.float32(0.123456)
    lo = float(np.float16(x)) if float(np.float16(x)) <= float(x) else float(
        np.nextafter(np.float16(x), np.float16(0)))
    hi = float(np.nextafter(np.float16(lo), np.float16(np.inf)))
    frac = (float(x) - lo) / (hi - lo)
    p = np.floor(128 * frac) / 128
    n = 4000
    got = np.array([oracle.sr_f16(np.array([x]), oracle.sr_bits(s, 1, 0, 1)).view(np.float16)[0]
                    for s in range(n)], np.float64)
    mean_up = np.mean(got == hi)
    assert abs(mean_up - p) <= 4 * np.sqrt(p * (1 - p) / n)


def _sep_case(state_dtype, seed):
    spec = synth.CacheSpec(num_slots=6, nheads=4, ngroups=2, state_dtype=state_dtype, separate=True)
    cache = synth.make_cache(spec, seed)
    step = synth.make_step(spec, 4, 3, seed + 1, 5)
    return spec, cache, step


def test_separate_steps_read_only_the_read_checkpoint(oracle):
    spec, cache, step = _sep_case("fp8", 71)
    out1, _ = oracle.replay_step(cache.copy(), step)
    c2 = cache.copy()
    c2.recur[:] = 0
    out2, _ = oracle.replay_step(c2, step)
    assert np.array_equal(out1, out2)


@pytest.mark.parametrize("state_dtype", ["fp8", "bf16"])
def test_separate_flush_closed_form(oracle, state_dtype):
    """Separate flush: the recurrence checkpoint becomes SR(fp32(closed-form
    state from the old recurrence checkpoint)) and the read checkpoint the
    nearest encoding of the same fp32 values; ring_start advances."""
    spec, cache, step = _sep_case(state_dtype, 81)
    c = cache.copy()
    oracle.replay_step(c, step)
    before = c.copy()
    k = np.array([min(int(p) + 2, spec.ring_len) for p in step.pnat], np.int32)
    seed = 987654321
    assert oracle.flush(c, step.slot_idx, k, step.A, seed) == 0
    agree = []
    for b in range(step.batch):
        slot = int(step.slot_idx[b])
        h0 = oracle.decode_recur(before, slot)
        for h in range(spec.nheads):
            seq = R.sequence(before, synth.StepInputs(**{**step.__dict__, "pnat": k}), b, h)
            want = R.closed_form_state(h0[h], float(step.A[h]), seq["dtp"][: k[b]], seq["x"][: k[b]],
                                       seq["B"][: k[b]]).astype(np.float32)
            u = oracle.sr_bits(seed, slot, h, spec.headdim * spec.dstate).reshape(spec.headdim, spec.dstate)
            sr_want = _sr_numpy(want, u)
            agree.append(np.mean(c.recur_logical(slot)[h] == sr_want))
            if state_dtype == "bf16":
                got = R.bf16_to_f64(c.state_logical(slot)[h])
                assert np.max(np.abs(got - want) / (1e-30 + np.abs(want))) <= 2.0 ** -8
    assert min(agree) >= 0.999, min(agree)
    assert np.array_equal(c.ring_start[step.slot_idx], (before.ring_start[step.slot_idx] + k) % spec.ring_len)


def test_separate_init_is_exact(oracle):
    spec = synth.CacheSpec(num_slots=5, nheads=3, ngroups=1, state_dtype="fp8", separate=True)
    cache = synth.make_cache(spec, 91)
    rng = np.random.default_rng(4)
    states = (rng.standard_normal((2, 3, 64, 128)) * 0.2).astype(np.float32)
    ids = np.array([2, 4], np.int32)
    oracle.init_state(cache, states, ids, seed=42)
    for j, slot in enumerate(ids):
        for h in range(3):
            u = oracle.sr_bits(42, int(slot), h, 64 * 128).reshape(64, 128)
            assert np.array_equal(cache.recur_logical(int(slot))[h], _sr_numpy(states[j, h], u))
