"""GPU parity of separate checkpoints (an FP16 recurrence checkpoint beside the
fp8 read checkpoint, stochastically rounded on every write).

vLLM PR "Add separate CuTeDSL ReplaySSM checkpoints" (Overview, Claims): the
recurrence checkpoint keeps FP16 with 7-bit stochastic rounding while steps
read the low-precision read checkpoint.  The random bits are Philox4x32-10 of
the call's seed, so the GPU and the oracle draw the same bits; they differ
only where the fp32 fold result and the oracle's fp64 one fall on opposite
sides of a rounding threshold.  Checked through the C ABI: init bit for bit,
flush and fused step against the oracle, the fused step against the GPU's own
flush-then-step bit for bit, steps that leave the recurrence checkpoint
alone, and several fold cycles in a row.

How a folded recurrence value is checked: for a fixed random u, stochastic
rounding is monotone in the value.  The oracle gives the exact fold v (fp64,
from a copy of the cache whose checkpoint holds the FP16 recurrence values)
and the fold of absolute values S (|h|, |x|, |B|; every coefficient is >= 0),
which bounds what fp32 arithmetic can move the sum: the kernel's products
use a two-term bf16 split of fp32 weights (relative error <= 2^-17) and
accumulate in fp32, so |v_gpu - v| <= 2^-15 S + 2^-23 |v|.  The GPU's fp16
bits must lie between SR(v - E, u) and SR(v + E, u), and most of them equal
SR(v, u).
"""
import numpy as np
import pytest
import torch

import synth
from synth import device as sd

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_harness as gh
    import speculative_replay_state_amd as ssu
from oracle import ssu_oracle as O


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _f16_ordinal(bits):
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def f16_agreement(got, ref):
    """(fraction equal, max distance in fp16 steps) of fp16 bit patterns; +-0 equal."""
    og, orf = _f16_ordinal(got), _f16_ordinal(ref)
    return float((og == orf).mean()), int(np.max(np.abs(og - orf))) if og.size else 0


SPECS = {
    "fp8_L16": dict(num_slots=40, nheads=32, ngroups=4),
    "fp8_L32": dict(num_slots=24, nheads=16, ngroups=2, ring_len=32),
}


def _spec(name, **kw):
    return synth.CacheSpec(state_dtype="fp8", separate=True, **{**SPECS[name], **kw})


def _fold_counts(step, seed):
    rng = np.random.default_rng(seed)
    k = np.array([rng.integers(0, int(p) + 1) for p in step.pnat], np.int32)
    k[int(np.argmax(step.pnat))] = int(np.max(step.pnat))
    return k


def test_separate_requires_fp8_state():
    spec = synth.CacheSpec(num_slots=4, nheads=8, ngroups=1, state_dtype="fp8", separate=True)
    cache = synth.make_cache(spec, 3)
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    dc.state_dtype = "bf16"
    ids = torch.zeros(1, dtype=torch.int32, device=gh.DEV)
    with pytest.raises(ssu.SsuError) as e:
        ssu.flush(dc, ids, ids, torch.zeros(8, device=gh.DEV))
    assert e.value.code == ssu.SSU_ERR_UNSUPPORTED


@pytest.mark.parametrize("broadcast", [False, True])
def test_separate_init_is_bit_exact(broadcast):
    spec = synth.CacheSpec(num_slots=12, nheads=16, ngroups=2, state_dtype="fp8", separate=True, slot_pad=64)
    cache = synth.make_cache(spec, 43)
    rng = np.random.default_rng(8)
    n = 6
    states = (rng.standard_normal((n, 16, 64, 128)) * 0.2).astype(np.float32)
    states[1, 3, 5, :] = 0.0
    states[2, 0, 0, 7] = 1e-39      # below the fp16 subnormal range
    states[2, 0, 1, :5] = [3e-5, -6.1e-5, 7e-8, 65504.0, 70000.0]  # fp16 subnormals, max, overflow
    ids = np.array([3, 0, 7, 12, 11, 1], np.int32)
    seed = 0x9E3779B97F4A7C15
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    ssu.init_state(dc, torch.from_numpy(states).to(gh.DEV), torch.from_numpy(ids).to(gh.DEV),
                   states_batch_stride=0 if broadcast else None, sr_seed=seed)
    torch.cuda.synchronize()
    ref = cache.copy()
    O.init_state(ref, states, ids, states_stride=0 if broadcast else None, seed=seed)
    gpu = sd.download_cache(spec, t)
    assert np.array_equal(gpu.recur, ref.recur)  # same Philox bits, exact fp32 inputs
    assert np.array_equal(gpu.scale, ref.scale)
    frac, dist = gh.fp8_code_agreement(gpu.state, ref.state)
    assert frac >= 0.999 and dist <= 1
    for f in ("x_cache", "B_cache", "dt_cache", "ring_start"):
        assert np.array_equal(getattr(gpu, f), getattr(ref, f)), f


@pytest.mark.parametrize("name", list(SPECS))
def test_separate_flush_parity(name):
    spec = _spec(name)
    cache = synth.make_cache(spec, 51)
    step = synth.make_step(spec, 20, 4, 52, 8)
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, "bf16")
    gh.run_step(dc, st, step, out, "bf16", "monolith")
    ref = cache.copy()
    O.replay_step(ref, step)
    rng = np.random.default_rng(9)
    k = np.array([rng.integers(0, int(p) + 5) for p in step.pnat], np.int32)
    k[0], k[1] = 0, min(int(step.pnat[1]) + 4, spec.ring_len)
    seed = 0xDEADBEEF12345678
    print("flush", name, "k", k[:8], flush=True)
    ssu.flush(dc, st["slot_idx"], torch.from_numpy(k).to(gh.DEV), st["A"], sr_seed=seed)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    before = ref.copy()
    assert O.flush(ref, step.slot_idx, k, step.A, seed) == 0
    gpu = sd.download_cache(spec, t)
    assert np.array_equal(gpu.ring_start, ref.ring_start)
    touched = sorted({int(s) for s, kk in zip(step.slot_idx, k) if kk > 0})
    gh.check_state(spec, gpu, ref, before, touched, (step.slot_idx, k, step.A))
    gh.check_recur(spec, gpu, before, step.slot_idx, k, step.A, seed)


def _run_fused(spec, cache, step, k, seed, with_z=False):
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, "bf16")
    desc = ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"],
                              st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, "bf16",
                              None, "auto", num_fold=torch.from_numpy(k).to(gh.DEV),
                              z=st.get("z") if with_z else None, sr_seed=seed)
    ssu.replay_step(dc, desc)
    torch.cuda.synchronize()
    return out, sd.download_cache(spec, t), int(dc.status.item())


@pytest.mark.parametrize("with_z", [False, True])
@pytest.mark.parametrize("name", list(SPECS))
def test_separate_fused_step_parity(name, with_z):
    spec = _spec(name)
    cache = synth.make_cache(spec, 61 + len(name))
    T = 8 if spec.ring_len > 16 else 4
    step = synth.make_step(spec, 17, T, 62, spec.ring_len - T, with_z=with_z)
    k = _fold_counts(step, 63)
    seed = 0x0123456789ABCDEF
    print("fused", name, with_z, "k", k[:8], flush=True)
    out, gpu, status = _run_fused(spec, cache, step, k, seed, with_z)
    assert status == 0
    ref_cache = cache.copy()
    ref, st = O.replay_step(ref_cache, step, num_fold=k, seed=seed)
    assert st == 0
    gh.check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, "bf16")
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
    assert np.array_equal(gpu.x_cache, ref_cache.x_cache)
    assert np.array_equal(gpu.B_cache, ref_cache.B_cache)
    touched = sorted({int(s) for s, kk in zip(step.slot_idx, k) if kk > 0 and 0 < s < spec.num_slots})
    gh.check_state(spec, gpu, ref_cache, cache, touched, (step.slot_idx, k, step.A))
    gh.check_recur(spec, gpu, cache, step.slot_idx, k, step.A, seed)


@pytest.mark.parametrize("name", list(SPECS))
def test_separate_fused_equals_gpu_flush_then_step(name):
    spec = _spec(name)
    cache = synth.make_cache(spec, 71)
    T = 8 if spec.ring_len > 16 else 4
    step = synth.make_step(spec, 19, T, 72, spec.ring_len - T)
    k = _fold_counts(step, 73)
    seed = 77
    out_f, gpu_f, st_f = _run_fused(spec, cache, step, k, seed)
    assert st_f == 0
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    st = sd.upload_step(step, gh.DEV)
    ssu.flush(dc, st["slot_idx"], torch.from_numpy(k).to(gh.DEV), st["A"], sr_seed=seed)
    step2 = synth.StepInputs(**{**step.__dict__, "pnat": (step.pnat - k).astype(np.int32)})
    st2 = sd.upload_step(step2, gh.DEV)
    out_s = gh.out_tensor(step, spec, "bf16")
    gh.run_step(dc, st2, step2, out_s, "bf16", "monolith")
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    gpu_s = sd.download_cache(spec, t)
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    for f in sd.CACHE_FIELDS + ("recur", "ring_start"):
        assert np.array_equal(getattr(gpu_f, f), getattr(gpu_s, f)), f


@pytest.mark.parametrize("algo", ["monolith", "split"])
def test_separate_plain_step_reads_only_the_read_checkpoint(algo):
    """Without a fold the step leaves the recurrence checkpoint alone and
    gives the same bits as the same cache without one."""
    spec = _spec("fp8_L16")
    cache = synth.make_cache(spec, 81)
    step = synth.make_step(spec, 12, 4, 82, 8)
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, "bf16")
    gh.run_step(dc, st, step, out, "bf16", algo)
    dc.recur = None
    out2 = gh.out_tensor(step, spec, "bf16")
    t2 = sd.upload_cache(cache, gh.DEV)
    dc2 = gh.device_cache(spec, t2)
    dc2.recur = None
    gh.run_step(dc2, st, step, out2, "bf16", algo)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    gpu = sd.download_cache(spec, t)
    assert np.array_equal(gpu.recur, cache.recur)
    assert np.array_equal(gpu.state, cache.state)


def _ulp16(x):
    """Spacing of fp16 values at |x| (2^-24 in the subnormal range)."""
    a = np.maximum(np.abs(x), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(a)) - 10)


def test_separate_fold_cycles():
    """Four rounds of fused step + fold with fresh inputs and seeds, the GPU
    and the oracle each on its own chain.  A fold scales the difference the
    two chains already had by beta <= 1 and adds at most the fp32 fold bound
    and two fp16 steps of stochastic rounding, so the bound on every
    recurrence value grows by that much per fold; most values stay equal."""
    spec = _spec("fp8_L16", num_slots=24)
    cache = synth.make_cache(spec, 91)
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    ref = cache.copy()
    slots = None
    bound = {}
    for cycle in range(4):
        step = synth.make_step(spec, 16, 4, 100 + cycle, 8, slots=slots)  # the same sequences every cycle
        slots = step.slot_idx.copy()
        k = _fold_counts(step, 200 + cycle)
        seed = 1000 + cycle
        print("cycle", cycle, flush=True)
        st = sd.upload_step(step, gh.DEV)
        out = gh.out_tensor(step, spec, "bf16")
        desc = ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"],
                                  st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, "bf16",
                                  None, "auto", num_fold=torch.from_numpy(k).to(gh.DEV), sr_seed=seed)
        ssu.replay_step(dc, desc)
        torch.cuda.synchronize()
        assert int(dc.status.item()) == 0
        s_abs = gh.f64_fold(spec, ref, slots, k, step.A, absolute=True)
        O.replay_step(ref, step, num_fold=k, seed=seed)
        gpu = sd.download_cache(spec, t)
        assert np.array_equal(gpu.ring_start, ref.ring_start)
        equal = total = 0
        for sl in sorted(int(x) for x in slots):
            g, r = O.decode_recur(gpu, sl), O.decode_recur(ref, sl)
            prev = bound.get(sl, 0.0)
            if sl in s_abs:
                bound[sl] = prev + 2 * _ulp16(r) + gh.FOLD_REL * s_abs[sl]
            over = np.abs(g - r) - bound.get(sl, 0.0)
            assert np.all(over <= 0), (cycle, sl, float(np.max(over)))
            equal += int((g == r).sum())
            total += g.size
        assert equal >= 0.97 * total, (cycle, equal / total)
