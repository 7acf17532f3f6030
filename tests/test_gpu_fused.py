"""GPU parity of the fused flush-in-step (replay step with num_fold).

The oracle defines the fused call as a flush of the first k live tokens
followed by the step with pnat - k.  Checked here on the GPU through the C
ABI: outputs against the oracle's plain step on the GPU's own post-fold
checkpoint at the plain bound, and against the oracle's composition (plus the
propagation of the accepted state differences); cache against the oracle's
flush (bounds as for the flush); the GPU's own flush-then-step bit for bit,
k = 0 against the plain monolith step bit for bit, and invalid k reported and
skipped.
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
from tests.test_gpu_replay import CASES, _setup


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _fold_counts(step, seed):
    """k ~ U{0..pnat}, with the entry of largest pnat folding its whole prefix."""
    rng = np.random.default_rng(seed)
    k = np.array([rng.integers(0, int(p) + 1) for p in step.pnat], np.int32)
    k[int(np.argmax(step.pnat))] = int(np.max(step.pnat))
    return k


def _run_fused(spec, cache, step, out_dtype, k, algo="auto"):
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, out_dtype)
    kt = torch.from_numpy(np.asarray(k, np.int32)).to(gh.DEV)
    desc = ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"],
                              st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, out_dtype,
                              None, algo, num_fold=kt)
    ssu.replay_step(dc, desc)
    torch.cuda.synchronize()
    return out, sd.download_cache(spec, t), int(dc.status.item())


@pytest.mark.parametrize("case", list(CASES))
def test_fused_step_parity(case):
    spec, cache, step, out_dtype = _setup(case, 3000 + len(case))
    k = _fold_counts(step, 7 + len(case))
    print("case", case, "k", k[:8], flush=True)
    out, gpu, status = _run_fused(spec, cache, step, out_dtype, k)
    assert status == 0
    ref_cache = cache.copy()
    ref, st = O.replay_step(ref_cache, step, num_fold=k)
    assert st == 0
    gh.check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, out_dtype)
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
    assert np.array_equal(gpu.x_cache, ref_cache.x_cache)
    assert np.array_equal(gpu.B_cache, ref_cache.B_cache)
    nb = spec.dt_bytes()
    gd = gpu.dt_cache[:, :nb].view(np.float32).astype(np.float64)
    rd = ref_cache.dt_cache[:, :nb].view(np.float32).astype(np.float64)
    assert gh.rel_err(gd, rd) <= 1e-6
    touched = sorted({int(s) for s, kk in zip(step.slot_idx, k) if kk > 0 and 0 < s < spec.num_slots})
    gh.check_state(spec, gpu, ref_cache, cache, touched, (step.slot_idx, k, step.A))


@pytest.mark.parametrize("case", list(CASES))
def test_fused_equals_gpu_flush_then_step(case):
    """One fused pass gives the same bits as the flush kernel then the step."""
    spec, cache, step, out_dtype = _setup(case, 4000 + len(case))
    k = _fold_counts(step, 11 + len(case))
    out_f, gpu_f, st_f = _run_fused(spec, cache, step, out_dtype, k)
    assert st_f == 0
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    st = sd.upload_step(step, gh.DEV)
    ssu.flush(dc, st["slot_idx"], torch.from_numpy(k).to(gh.DEV), st["A"])
    step2 = synth.StepInputs(**{**step.__dict__, "pnat": (step.pnat - k).astype(np.int32)})
    st2 = sd.upload_step(step2, gh.DEV)
    out_s = gh.out_tensor(step, spec, out_dtype)
    gh.run_step(dc, st2, step2, out_s, out_dtype, "monolith")
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    gpu_s = sd.download_cache(spec, t)
    view = torch.int32 if out_f.dtype == torch.float32 else torch.int16
    assert torch.equal(out_f.view(view), out_s.view(view))
    for f in sd.CACHE_FIELDS:
        assert np.array_equal(getattr(gpu_f, f), getattr(gpu_s, f)), f


@pytest.mark.parametrize("case", ["mtp_bf16", "fp8", "f32_T16_L32"])
def test_fused_k0_equals_plain_step(case):
    spec, cache, step, out_dtype = _setup(case, 5000 + len(case))
    k = np.zeros(step.batch, np.int32)
    out_f, gpu_f, st_f = _run_fused(spec, cache, step, out_dtype, k)
    assert st_f == 0
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    st = sd.upload_step(step, gh.DEV)
    out_s = gh.out_tensor(step, spec, out_dtype)
    gh.run_step(dc, st, step, out_s, out_dtype, "monolith")
    torch.cuda.synchronize()
    view = torch.int32 if out_f.dtype == torch.float32 else torch.int16
    assert torch.equal(out_f.view(view), out_s.view(view))
    gpu_s = sd.download_cache(spec, t)
    for f in sd.CACHE_FIELDS:
        assert np.array_equal(getattr(gpu_f, f), getattr(gpu_s, f)), f


def test_fused_invalid_fold_is_skipped_and_reported():
    spec = synth.CacheSpec(num_slots=16, nheads=16, ngroups=2, state_dtype="fp8")
    cache = synth.make_cache(spec, 61)
    step = synth.make_step(spec, 6, 3, 62, 6)
    step.pnat[:] = [3, 2, 4, 0, 5, 1]
    k = np.array([2, 3, -1, 0, 5, 1], np.int32)  # entries 1 (k > pnat) and 2 (k < 0) invalid
    out, gpu, status = _run_fused(spec, cache, step, "bf16", k)
    assert status == ssu.SSU_STATUS_BAD_FOLD
    ref_cache = cache.copy()
    ref, st = O.replay_step(ref_cache, step, num_fold=k)
    assert st == ssu.SSU_STATUS_BAD_FOLD
    got = gh.to_f64(out)
    assert np.all(got[3:9] == 0.0)
    gh.check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, "bf16")
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
    for b in (1, 2):
        s = int(step.slot_idx[b])
        assert np.array_equal(gpu.state[s], cache.state[s])
        assert np.array_equal(gpu.x_cache[s], cache.x_cache[s])
    touched = sorted({int(step.slot_idx[b]) for b in (0, 4, 5)})
    k_valid = np.where((k >= 0) & (k <= step.pnat), k, 0).astype(np.int32)
    gh.check_state(spec, gpu, ref_cache, cache, touched, (step.slot_idx, k_valid, step.A))


def _scaled_bf16(bits, factor):
    """bf16 bits times a power of two (exact while in range)."""
    v = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kind", ["flush", "fused"])
def test_fp8_fold_extreme_rows(kind):
    """fp8 folds far from unit scale, against the oracle.  With f = D0 *
    old_scale the per-row decay of the old codes: slot 2 (row scales 2^-70)
    has f < 2^-60 and new scales near 2^-10; slot 3 (scales 2^-40, ring x
    and B times 2^50) folds values near 2^100 into rows whose old values are
    below 2^-30; slot 4 (scales 2^59, ring x and B times 2^58) gets new
    scales above 2^100, outside the fast reciprocal encode's range.  Slots 1
    and 5 are ordinary."""
    spec = synth.CacheSpec(num_slots=8, nheads=16, ngroups=2, state_dtype="fp8")
    cache = synth.make_cache(spec, 97)
    cache.scale_view(2)[:] = np.float32(2.0 ** -70)
    cache.scale_view(3)[:] = np.float32(2.0 ** -40)
    cache.scale_view(4)[:] = np.float32(2.0 ** 59)
    for sl, e in ((3, 50), (4, 58)):
        cache.x_view(sl)[:] = _scaled_bf16(cache.x_view(sl), 2.0 ** e)
        cache.B_view(sl)[:] = _scaled_bf16(cache.B_view(sl), 2.0 ** e)
    slots = np.array([1, 2, 3, 4, 5], np.int32)
    step = synth.make_step(spec, 5, 4, 98, 8, slots=slots)
    step.pnat[:] = [6, 8, 8, 8, 5]
    k = step.pnat.copy()
    print("fp8 extreme rows", kind, flush=True)
    ref_cache = cache.copy()
    if kind == "flush":
        t = sd.upload_cache(cache, gh.DEV)
        st = sd.upload_step(step, gh.DEV)
        dc = gh.device_cache(spec, t)
        ssu.flush(dc, st["slot_idx"], torch.from_numpy(k).to(gh.DEV), st["A"])
        torch.cuda.synchronize()
        assert int(dc.status.item()) == 0
        gpu = sd.download_cache(spec, t)
        assert O.flush(ref_cache, step.slot_idx, k, step.A) == 0
    else:
        out, gpu, status = _run_fused(spec, cache, step, "bf16", k)
        assert status == 0
        ref, st_ = O.replay_step(ref_cache, step, num_fold=k)
        assert st_ == 0
        gh.check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, "bf16")
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
    sc = [gpu.scale_view(s).astype(np.float64) for s in (2, 3, 4)]
    assert np.min(sc[1]) > 2.0 ** 70 and np.median(sc[2]) > 2.0 ** 100, (np.min(sc[1]), np.median(sc[2]))
    gh.check_state(spec, gpu, ref_cache, cache, [1, 2, 3, 4, 5], (step.slot_idx, k, step.A))


def _with_empty_entries(step, empty):
    """The varlen step with the entries in `empty` given no new tokens."""
    cu = step.cu_seqlens
    tb = np.diff(cu).astype(np.int32)
    tb[empty] = 0
    rows = np.concatenate([np.arange(cu[b], cu[b] + tb[b]) for b in range(step.batch)]).astype(np.int64)
    cu2 = np.zeros(step.batch + 1, np.int32)
    cu2[1:] = np.cumsum(tb)
    return synth.StepInputs(**{**step.__dict__, "cu_seqlens": cu2, "x": step.x[rows], "B": step.B[rows],
                               "C": step.C[rows], "dt": step.dt[rows]})


@pytest.mark.parametrize("state_dtype", ["fp8", "f16"])
def test_fused_empty_windows(state_dtype):
    """Varlen entries without new tokens: some fold their whole live prefix
    (an empty readout window after the fold), some have nothing live either,
    one is the last entry (its first row is the end of the packed inputs).
    Against the oracle, and bit for bit against the GPU's flush then step."""
    spec = synth.CacheSpec(num_slots=40, nheads=32, ngroups=4, state_dtype=state_dtype)
    cache = synth.make_cache(spec, 6100)
    step = synth.make_step(spec, 12, 4, 6101, 6, varlen=True)
    step.pnat[[1, 4, 11]] = [5, 3, 2]
    step.pnat[7] = 0
    step = _with_empty_entries(step, [1, 4, 7, 11])
    k = _fold_counts(step, 6102)
    k[[1, 4, 11]] = step.pnat[[1, 4, 11]]  # fold everything live: nothing left to read out
    k[7] = 0
    print("case empty windows", state_dtype, "Tb", np.diff(step.cu_seqlens), "pnat", step.pnat, "k", k, flush=True)
    out, gpu, status = _run_fused(spec, cache, step, "bf16", k)
    assert status == 0
    ref_cache = cache.copy()
    ref, st = O.replay_step(ref_cache, step, num_fold=k)
    assert st == 0
    gh.check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, "bf16")
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
    assert np.array_equal(gpu.x_cache, ref_cache.x_cache)
    assert np.array_equal(gpu.B_cache, ref_cache.B_cache)
    touched = sorted({int(s) for s, kk in zip(step.slot_idx, k) if kk > 0 and 0 < s < spec.num_slots})
    gh.check_state(spec, gpu, ref_cache, cache, touched, (step.slot_idx, k, step.A))
    # the same bits as the flush kernel followed by the plain step
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    st_in = sd.upload_step(step, gh.DEV)
    ssu.flush(dc, st_in["slot_idx"], torch.from_numpy(k).to(gh.DEV), st_in["A"])
    step2 = synth.StepInputs(**{**step.__dict__, "pnat": (step.pnat - k).astype(np.int32)})
    st2 = sd.upload_step(step2, gh.DEV)
    out_s = gh.out_tensor(step, spec, "bf16")
    gh.run_step(dc, st2, step2, out_s, "bf16", "monolith")
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    assert torch.equal(out.view(torch.int16), out_s.view(torch.int16))
    gpu_s = sd.download_cache(spec, t)
    for f in sd.CACHE_FIELDS:
        assert np.array_equal(getattr(gpu, f), getattr(gpu_s, f)), f
